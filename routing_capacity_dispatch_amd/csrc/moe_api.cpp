// Host side of the C ABI: validation, capacity plan, workspace carving and
// the launch sequence of the branch.  No allocation, no host synchronisation.
#include "moe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kI32Max = 2147483647;
constexpr int32_t kMaxWidth = 1 << 20;  // largest d_model, d_latent, d_ff, d_ff_shared
// Most entries of a grouped GEMM's tile list: its grid (one 512-thread
// workgroup per entry, rounded up to a multiple of 8) stays below 2^32
// work-items.
constexpr int64_t kMaxListEntries = (int64_t(1) << 23) - 8;

// Stages of moe_forward, in launch order: latent GEMM, router GEMM, top-k,
// slot assignment, row scatter, receiver binning, expert row lists, expert
// gate/up GEMM, expert down GEMM, combine, shared gate/up GEMM, output GEMM.
constexpr int kStages = 12;

// Records stage boundary i (event i) on the stream when events are given.
struct Marks {
  void* const* ev;
  int n;
  int next;
  hipError_t mark(hipStream_t s) {
    if (!ev || next >= n) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[next++]), s);
  }
};


int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  int64_t used;
  void* take(int64_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align256(bytes);
    return p;
  }
};

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

// Sizes every entry point needs.  top_k is the number of assignments per
// token; only selection (moe_route, moe_forward) also needs top_k <= E.
moe_status check_route_shape(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->n_experts < 1 || c->top_k < 1) return MOE_ERR_INVALID_ARG;
  if (c->T * (int64_t)c->n_experts > kI32Max * 64) return MOE_ERR_UNSUPPORTED;
  if (c->T * (int64_t)c->top_k > kI32Max) return MOE_ERR_INVALID_ARG;
  if (c->n_experts > 1024 || c->top_k > 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Capacity with exact integer arithmetic: ceil(num * Tw * k / (den * n)).
int64_t capacity(int64_t num, int64_t den, int64_t Tw, int64_t k, int64_t n) {
  const __int128 a = (__int128)num * Tw * k;
  const __int128 b = (__int128)den * n;
  return (int64_t)((a + b - 1) / b);
}

// The routed experts' grouped GEMMs take 256-row tiles instead of 192-row
// ones when an expert's expected rows ceil(T k / E) reach kTallRows: both
// tiles then pad an expert by a few per cent at most, and the taller tile
// does more MFMA work per staged operand byte.  A function of the config
// only, so the plan's workspace sizes and every launch agree.
constexpr int64_t kTallRows = 4096;
bool tall_tiles(const moe_config* c) {
  return ceil_div(c->T * (int64_t)c->top_k, c->n_experts) >= kTallRows;
}

// Upper bounds of the ragged GEMMs' tile lists: expert e has
// ceil(count_e / bm) <= count_e / bm + 1 M tiles.
void dropless_entries(const moe_config* c, int64_t* ent0, int64_t* ent1) {
  const int64_t n = c->T * (int64_t)c->top_k;
  const int64_t bm = moe::ragged_tile_rows(tall_tiles(c));
  const int64_t mt = ceil_div(n, bm) + c->n_experts;
  *ent0 = mt * ceil_div(c->d_ff, moe::ragged_gate_up_cols());
  *ent1 = mt * ceil_div(c->d_latent, moe::ragged_down_cols());
}

// Tile-list bounds of the capped path's grouped GEMMs: expert e holds at
// most max_rows kept rows, and sum_e count_e <= E * max_rows.
void capped_entries(const moe_config* c, int64_t max_rows, int64_t* ent0, int64_t* ent1) {
  const int64_t bm = moe::ragged_tile_rows(tall_tiles(c));
  const int64_t E = c->n_experts;
  const int64_t per = ceil_div(max_rows, bm);
  const int64_t mt = per * E < ceil_div(E * max_rows, bm) + E ? per * E : ceil_div(E * max_rows, bm) + E;
  *ent0 = mt * ceil_div(c->d_ff, moe::ragged_gate_up_cols());
  *ent1 = mt * ceil_div(c->d_latent, moe::ragged_down_cols());
}

// Tile-list bounds of the backward's grouped dgrad GEMMs over R padded
// rows: sum_e ceil(rows_e / bm) <= R / bm + E M tiles.
void backward_entries(const moe_config* c, int64_t R, int64_t* pre, int64_t* dh, int64_t* du) {
  const int64_t mt = ceil_div(R, moe::bwd_dgrad_rows()) + c->n_experts;
  *pre = mt * ceil_div(c->d_ff, moe::ragged_gate_up_cols());
  *dh = mt * ceil_div(c->d_ff, moe::bwd_dgrad_cols());
  *du = mt * ceil_div(c->d_latent, moe::bwd_dgrad_cols());
}

moe_status plan_impl(const moe_config* c, moe_plan* p) {
  if (!c || !p) return MOE_ERR_INVALID_ARG;
  moe_status st = check_route_shape(c);
  if (st != MOE_OK) return st;
  if (c->d_model < 1 || c->d_latent < 1 || c->d_ff < 1 || c->n_pools < 1 || c->n_waves < 1 ||
      c->n_shared < 0 || (c->n_shared > 0 && c->d_ff_shared < 1))
    return MOE_ERR_INVALID_ARG;
  if (c->n_experts % c->n_pools) return MOE_ERR_INVALID_ARG;
  if (c->send_cap_num < 0 || c->send_cap_den < 1 || c->recv_cap_num < 0 || c->recv_cap_den < 1 ||
      c->cap_send_rows < 0 || c->cap_recv_rows < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (c->d_model % 64 || c->d_latent % 64 || c->d_ff % 64 ||
      (c->n_shared > 0 && c->d_ff_shared % 64))
    return MOE_ERR_UNSUPPORTED;
  // widths up to 2^20: with T * k < 2^31 and every capacity product below
  // 2^31, each workspace size below stays far inside int64
  if (c->d_model > kMaxWidth || c->d_latent > kMaxWidth || c->d_ff > kMaxWidth ||
      (c->n_shared > 0 && c->d_ff_shared > kMaxWidth))
    return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 3) return MOE_ERR_UNSUPPORTED;
  if (c->n_waves > 65535) return MOE_ERR_UNSUPPORTED;  // the slot scan's grid has one row per wave

  const int64_t T = c->T, W = c->n_waves, E = c->n_experts, P = c->n_pools, k = c->top_k;
  const int64_t Tw = ceil_div(T, W);
  const int64_t cs = c->cap_send_rows ? c->cap_send_rows
                                      : capacity(c->send_cap_num, c->send_cap_den, Tw, k, P);
  const int64_t cr = c->cap_recv_rows ? c->cap_recv_rows
                                      : capacity(c->recv_cap_num, c->recv_cap_den, Tw, k, E);
  // every index the kernels form stays inside int32 (each capacity first, so
  // no product can overflow: W, P, E < 2^17)
  if (cs > kI32Max || cr > kI32Max || W * P * cs > kI32Max || W * E * cr > kI32Max)
    return MOE_ERR_UNSUPPORTED;
  const int64_t eb = c->dtype == MOE_BF16 ? 2 : 4;
  const int64_t L = c->d_latent, F = c->d_ff;
  const int64_t S = c->n_shared, Fs = c->d_ff_shared;

  // the bf16 GEMMs address each operand buffer as a scalar base plus a
  // 32-bit lane offset: every buffer read from one base stays below 4 GiB
  if (c->dtype == MOE_BF16) {
    const int64_t kLim = int64_t(1) << 32;
    const int64_t D = c->d_model;
    const int64_t pools = W * P * align256(cs * L * 2 + cs * 4);
    const int64_t widest = D > L ? D : L;
    if (T * widest * 2 >= kLim || T * S * Fs * 2 >= kLim || pools >= kLim || F * L * 2 >= kLim ||
        L * D * 2 >= kLim || Fs * D * 2 >= kLim)
      return MOE_ERR_UNSUPPORTED;
  }

  p->tokens_per_wave = Tw;
  p->cap_send = cs;
  p->cap_recv = cr;
  p->experts_per_pool = E / P;
  p->elem_bytes = eb;
  p->row_bytes = L * eb;
  p->ids_offset = cs * L * eb;
  p->pool_block_bytes = align256(p->ids_offset + cs * 4);
  p->pools_bytes = W * P * p->pool_block_bytes;
  p->expert_out_bytes = align256(W * P * cs * L * eb);
  p->max_expert_rows = W * cr;

  Carver d{nullptr, 0};
  d.take(W * 3 * 8);  // per-wave counters
  d.take(W * moe::assign_chunks(Tw, k) * (int64_t)(E + P) * 4);  // per-chunk key counts of the slot scan
  p->dispatch_ws_bytes = d.used;

  Carver x{nullptr, 0};
  if (c->dtype == MOE_BF16) {
    int64_t e0, e1;
    capped_entries(c, W * cr, &e0, &e1);
    if (e0 > kMaxListEntries || e1 > kMaxListEntries) return MOE_ERR_UNSUPPORTED;
    x.take((E + 1) * 4);          // expert-major row offsets
    x.take(E * W * cr * 4);       // flat pool-row index of each kept row
    x.take(e0 * 12);              // gate/up tile list
    x.take(e1 * 12);              // down tile list
    x.take(8);                    // list lengths
    x.take(E * W * cr * F * eb);  // SwiGLU hidden rows, expert-major
  } else {
    x.take(E * W * cr * 4);       // expert row lists
    x.take(E * 4);                // rows per expert
    x.take(E * W * cr * F * eb);  // SwiGLU hidden rows
  }
  p->experts_ws_bytes = x.used;

  Carver f{nullptr, 0};
  f.take(T * L * eb);         // z
  f.take(T * E * 4);          // logits
  f.take(T * k * 4);          // topk
  f.take(T * k * 4);          // gates
  f.take(T * k * 4);          // pool_slot
  f.take(T * k * 4);          // recv_slot
  f.take(W * P * 4);          // pool_count
  f.take(W * E * 4);          // expert_count
  f.take(W * E * cr * 4);     // bank_rows
  f.take(p->pools_bytes);     // pools
  f.take(p->expert_out_bytes);
  f.take(T * L * eb);         // y_latent
  f.take(T * S * Fs * eb);    // shared hidden
  f.take(3 * 8);              // counters
  f.take(p->dispatch_ws_bytes);
  f.take(p->experts_ws_bytes);
  p->forward_ws_bytes = f.used;

  // dropless ragged variant
  const int64_t n = T * k;
  int64_t ent0, ent1;
  dropless_entries(c, &ent0, &ent1);
  if (ent0 > kMaxListEntries || ent1 > kMaxListEntries) return MOE_ERR_UNSUPPORTED;
  const int64_t nblk = moe::ragged_sort_blocks(n);
  p->dropless_rows = n;
  Carver dd{nullptr, 0};
  dd.take(nblk * E * 4);  // per-chunk histograms
  dd.take(nblk * E * 4);  // per-chunk bases
  p->dropless_dispatch_ws_bytes = dd.used;
  Carver dx{nullptr, 0};
  dx.take(ent0 * 12);     // gate/up tile list
  dx.take(ent1 * 12);     // down tile list
  dx.take(8);             // list lengths
  dx.take(n * F * eb);    // SwiGLU hidden rows
  p->dropless_experts_ws_bytes = dx.used;
  Carver df{nullptr, 0};
  df.take(T * L * eb);    // z
  df.take(T * E * 4);     // logits
  df.take(T * k * 4);     // topk
  df.take(T * k * 4);     // gates
  df.take(T * k * 4);     // row_of
  df.take((E + 1) * 4);   // expert offsets
  df.take(n * L * eb);    // xs
  df.take(n * L * eb);    // expert_out
  df.take(T * L * eb);    // y_latent
  df.take(T * S * Fs * eb);
  df.take(3 * 8);
  df.take(p->dropless_dispatch_ws_bytes);
  df.take(p->dropless_experts_ws_bytes);
  p->dropless_forward_ws_bytes = df.used;

  // backward of the routed path: expert e's kept rows, rounded up to 64
  const int64_t kept_max = T * k < E * W * cr ? T * k : E * W * cr;
  const int64_t R = kept_max + 63 * E;
  int64_t bpre, bdh, bdu;
  backward_entries(c, R, &bpre, &bdh, &bdu);
  if (R > kI32Max || bpre > kMaxListEntries || bdh > kMaxListEntries || bdu > kMaxListEntries)
    return MOE_ERR_UNSUPPORTED;
  p->backward_rows = R;
  Carver bx{nullptr, 0};
  bx.take(E * 4);           // rows per expert
  bx.take((E + 1) * 4);     // padded offsets
  bx.take(R * 4);           // pool row of each padded row
  bx.take(bpre * 12);       // recompute tile list
  bx.take(bdh * 12);        // dh tile list
  bx.take(bdu * 12);        // du tile list
  bx.take(16);              // list lengths
  bx.take(R * L * 2);       // u rows
  bx.take(R * L * 2);       // do rows
  bx.take(R * F * 2);       // dh
  bx.take(R * 2 * F * 2);   // da | db
  bx.take(R * F * 2);       // h
  p->experts_bwd_ws_bytes = bx.used;
  // ... and for the dropless variant, over its T*k rows
  const int64_t Rd = n + 63 * E;
  int64_t dpre, ddh, ddu;
  backward_entries(c, Rd, &dpre, &ddh, &ddu);
  if (Rd > kI32Max || dpre > kMaxListEntries || ddh > kMaxListEntries || ddu > kMaxListEntries)
    return MOE_ERR_UNSUPPORTED;
  p->dropless_backward_rows = Rd;
  Carver dbx{nullptr, 0};
  dbx.take(E * 4);
  dbx.take((E + 1) * 4);
  dbx.take(Rd * 4);
  dbx.take(dpre * 12);
  dbx.take(ddh * 12);
  dbx.take(ddu * 12);
  dbx.take(16);
  dbx.take(Rd * L * 2);
  dbx.take(Rd * L * 2);
  dbx.take(Rd * F * 2);
  dbx.take(Rd * 2 * F * 2);
  dbx.take(Rd * F * 2);
  p->dropless_experts_bwd_ws_bytes = dbx.used;
  Carver dbb{nullptr, 0};
  dbb.take(T * k * 4);       // d_gates
  dbb.take(n * L * eb);      // d_expert_out
  dbb.take(n * L * eb);      // d_xs
  dbb.take(p->dropless_experts_bwd_ws_bytes);
  p->dropless_backward_ws_bytes = dbb.used;
  Carver bb{nullptr, 0};
  bb.take(T * k * 4);              // d_gates
  bb.take(p->expert_out_bytes);    // d_expert_out
  bb.take(p->expert_out_bytes);    // d_pool_rows
  bb.take(p->experts_bwd_ws_bytes);
  p->backward_ws_bytes = bb.used;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe::DispatchArgs dispatch_args(const moe_config* c, const moe_plan& p, const int32_t* topk,
                                void* pools, int32_t* pool_slot, int32_t* recv_slot,
                                int32_t* pool_count, int64_t* wave_counts, int64_t* counts) {
  moe::DispatchArgs a{};
  a.topk = topk;
  a.T = c->T;
  a.k = c->top_k;
  a.E = c->n_experts;
  a.P = c->n_pools;
  a.W = c->n_waves;
  a.Tw = p.tokens_per_wave;
  a.cap_send = p.cap_send;
  a.cap_recv = p.cap_recv;
  a.pool_slot = pool_slot;
  a.recv_slot = recv_slot;
  a.pool_count = pool_count;
  a.pools = static_cast<char*>(pools);
  a.block_bytes = p.pool_block_bytes;
  a.ids_offset = p.ids_offset;
  a.row_bytes = p.row_bytes;
  a.wave_counts = wave_counts;
  a.counts = counts;
  return a;
}

moe_status run_dispatch(const moe_config* c, const moe_plan& p, const int32_t* topk, const void* z,
                        void* pools, int32_t* pool_slot, int32_t* recv_slot, int32_t* bank_rows,
                        int32_t* pool_count, int32_t* expert_count, int64_t* counts, void* ws,
                        hipStream_t s, Marks* m) {
  Carver cv{static_cast<char*>(ws), 0};
  int64_t* wave_counts = static_cast<int64_t*>(cv.take(c->n_waves * 3 * 8));
  moe::DispatchArgs a =
      dispatch_args(c, p, topk, pools, pool_slot, recv_slot, pool_count, wave_counts, counts);
  a.n_chunks = moe::assign_chunks(p.tokens_per_wave, c->top_k);
  a.chunk_counts = static_cast<int32_t*>(
      cv.take(c->n_waves * (int64_t)a.n_chunks * (c->n_experts + c->n_pools) * 4));
  hipError_t e = moe::launch_assign(a, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e == hipSuccess) e = moe::launch_scatter_rows(a, z, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e == hipSuccess) e = moe::launch_recv_bin(a, bank_rows, expert_count, s);
  if (e == hipSuccess && m) e = m->mark(s);
  return hip_status(e);
}

moe_status run_experts(const moe_config* c, const moe_plan& p, const void* pools,
                       const int32_t* bank_rows, const int32_t* expert_count, const void* wg,
                       const void* wu, const void* wd, void* expert_out, void* ws,
                       hipStream_t s, Marks* m) {
  const int E = c->n_experts;
  const int max_rows = (int)p.max_expert_rows;
  Carver cv{static_cast<char*>(ws), 0};
  if (c->dtype == MOE_BF16) {
    // expert-major row lists, then the grouped GEMMs over device-built tile
    // lists (rows gathered from the pools, outputs scattered back to them)
    int64_t ent0, ent1;
    capped_entries(c, max_rows, &ent0, &ent1);
    int32_t* offsets = static_cast<int32_t*>(cv.take((int64_t)(E + 1) * 4));
    int32_t* gidx = static_cast<int32_t*>(cv.take((int64_t)E * max_rows * 4));
    int32_t* list0 = static_cast<int32_t*>(cv.take(ent0 * 12));
    int32_t* list1 = static_cast<int32_t*>(cv.take(ent1 * 12));
    int32_t* ntiles = static_cast<int32_t*>(cv.take(8));
    char* H = static_cast<char*>(cv.take((int64_t)E * max_rows * c->d_ff * p.elem_bytes));
    const int tn0 = (int)ceil_div(c->d_ff, moe::ragged_gate_up_cols());
    const int tn1 = (int)ceil_div(c->d_latent, moe::ragged_down_cols());
    hipError_t e = moe::launch_expert_gidx(bank_rows, expert_count, E, c->n_pools, c->n_waves, p.cap_send,
                                           p.cap_recv, offsets, gidx, s);
    if (e == hipSuccess)
      e = moe::launch_ragged_tiles(offsets, E, moe::ragged_tile_rows(tall_tiles(c)), tn0, tn1, list0, list1,
                                   ntiles, s);
    if (e == hipSuccess && m) e = m->mark(s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    moe::RaggedGemm g{};
    g.A = static_cast<const char*>(pools);
    g.a_row_bytes = p.row_bytes;
    g.a_index = gidx;
    g.a_block_rows = (int)p.cap_send;
    g.a_block_bytes = p.pool_block_bytes;
    g.offsets = offsets;
    g.list = list0;
    g.ntiles = ntiles;
    g.W0 = static_cast<const char*>(wg);
    g.W1 = static_cast<const char*>(wu);
    g.E = E;
    g.F = c->d_ff;
    g.K = c->d_latent;
    g.C = H;
    g.c_row_bytes = (int64_t)c->d_ff * p.elem_bytes;
    e = moe::launch_ragged_gate_up_bf16(g, ent0, tall_tiles(c), s);
    if (e == hipSuccess && m) e = m->mark(s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    moe::RaggedGemm d{};
    d.A = H;
    d.a_row_bytes = (int64_t)c->d_ff * p.elem_bytes;
    d.offsets = offsets;
    d.list = list1;
    d.ntiles = ntiles + 1;
    d.W0 = static_cast<const char*>(wd);
    d.E = E;
    d.K = c->d_ff;
    d.N = c->d_latent;
    d.C = static_cast<char*>(expert_out);
    d.c_row_bytes = p.row_bytes;
    d.c_index = gidx;
    e = moe::launch_ragged_down_bf16(d, ent1, tall_tiles(c), s);
    if (e == hipSuccess && m) e = m->mark(s);
    return hip_status(e);
  }
  int32_t* erow = static_cast<int32_t*>(cv.take((int64_t)E * max_rows * 4));
  int32_t* rows_total = static_cast<int32_t*>(cv.take((int64_t)E * 4));
  void* H = cv.take((int64_t)E * max_rows * c->d_ff * p.elem_bytes);
  hipError_t e = moe::launch_expert_rows(bank_rows, expert_count, E, c->n_pools, c->n_waves,
                                         p.cap_send, p.cap_recv, erow, rows_total, max_rows, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::ExpertGateUp gu{};
  gu.pools = static_cast<const char*>(pools);
  gu.block_bytes = p.pool_block_bytes;
  gu.row_bytes = p.row_bytes;
  gu.cap_send = (int)p.cap_send;
  gu.erow = erow;
  gu.rows_total = rows_total;
  gu.E = E;
  gu.max_rows = max_rows;
  gu.F = c->d_ff;
  gu.L = c->d_latent;
  gu.Wg = wg;
  gu.Wu = wu;
  gu.H = H;
  e = moe::launch_expert_gate_up(c->dtype, gu, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::ExpertDown dn{};
  dn.H = H;
  dn.erow = erow;
  dn.rows_total = rows_total;
  dn.E = E;
  dn.max_rows = max_rows;
  dn.F = c->d_ff;
  dn.L = c->d_latent;
  dn.Wd = wd;
  dn.out = expert_out;
  e = moe::launch_expert_down(c->dtype, dn, s);
  if (e == hipSuccess && m) e = m->mark(s);
  return hip_status(e);
}

moe_status run_combine(const moe_config* c, const moe_plan& p, const void* expert_out,
                       const int32_t* topk, const int32_t* pool_slot, const int32_t* recv_slot,
                       const float* gates, void* y_latent, hipStream_t s, int64_t y_pitch = 0) {
  moe::CombineArgs a{};
  a.expert_out = static_cast<const char*>(expert_out);
  a.topk = topk;
  a.pool_slot = pool_slot;
  a.recv_slot = recv_slot;
  a.gates = gates;
  a.T = c->T;
  a.Tw = p.tokens_per_wave;
  a.k = c->top_k;
  a.E = c->n_experts;
  a.P = c->n_pools;
  a.cap_send = p.cap_send;
  a.row_bytes = p.row_bytes;
  a.y = y_latent;
  a.y_pitch = y_pitch;
  return hip_status(moe::launch_combine(c->dtype, a, s));
}

}  // namespace

MOE_API const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported shape";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small or misaligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
  }
  return "unknown moe_status";
}

MOE_API int32_t moe_version(void) { return 100; }

MOE_API moe_status moe_make_plan(const moe_config* cfg, moe_plan* plan) {
  return plan_impl(cfg, plan);
}

MOE_API moe_status moe_route(const moe_config* cfg, const float* logits, const float* bias,
                             int32_t* topk_idx, float* gates, void* stream) {
  moe_status st = check_route_shape(cfg);
  if (st != MOE_OK) return st;
  if (cfg->top_k > cfg->n_experts) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!logits || !topk_idx || !gates)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_topk_gates(logits, bias, cfg->T, cfg->n_experts, cfg->top_k,
                                           topk_idx, gates, static_cast<hipStream_t>(stream)));
}

static moe_status check_bias_update(const moe_config* cfg, int32_t n_bins) {
  moe_status st = check_route_shape(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T < 1 || cfg->top_k > cfg->n_experts) return MOE_ERR_INVALID_ARG;
  if (n_bins < 1 || n_bins > moe::bias_max_bins()) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

MOE_API moe_status moe_router_bias_ws_bytes(const moe_config* cfg, int32_t n_bins, size_t* bytes) {
  moe_status st = check_bias_update(cfg, n_bins);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = (size_t)moe::bias_ws_bytes(cfg->T, cfg->n_experts, n_bins);
  return MOE_OK;
}

static moe_status bias_update_impl(const moe_config* cfg, const float* logits, int32_t n_bins, float* bias_next,
                                   int32_t* hist, float* lohi, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events) {
  moe_status st = check_bias_update(cfg, n_bins);
  if (st != MOE_OK) return st;
  if (!logits || !bias_next) return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned256(ws) || (int64_t)ws_bytes < moe::bias_ws_bytes(cfg->T, cfg->n_experts, n_bins))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_bias_update(logits, cfg->T, cfg->n_experts, cfg->top_k, n_bins, bias_next, hist,
                                            lohi, ws, static_cast<hipStream_t>(stream), events));
}

MOE_API moe_status moe_router_bias_update(const moe_config* cfg, const float* logits, int32_t n_bins,
                                          float* bias_next, int32_t* hist, float* lohi, void* ws,
                                          size_t ws_bytes, void* stream) {
  return bias_update_impl(cfg, logits, n_bins, bias_next, hist, lohi, ws, ws_bytes, stream, nullptr);
}

MOE_API int32_t moe_router_bias_stage_count(void) { return 4; }

MOE_API moe_status moe_router_bias_update_profiled(const moe_config* cfg, const float* logits, int32_t n_bins,
                                                   float* bias_next, int32_t* hist, float* lohi, void* ws,
                                                   size_t ws_bytes, void* stream, void* const* stage_events,
                                                   int32_t n_events) {
  if (!stage_events || n_events < 5) return MOE_ERR_INVALID_ARG;
  return bias_update_impl(cfg, logits, n_bins, bias_next, hist, lohi, ws, ws_bytes, stream, stage_events);
}

MOE_API moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const void* z,
                                void* pools, int32_t* pool_slot, int32_t* recv_slot,
                                int32_t* bank_rows, int32_t* pool_count, int32_t* expert_count,
                                int64_t* counts, void* ws, size_t ws_bytes, void* stream) {
  moe_plan p;
  moe_status st = plan_impl(cfg, &p);
  if (st != MOE_OK) return st;
  if (!pool_count || !expert_count || !counts) return MOE_ERR_INVALID_ARG;
  if ((p.pools_bytes > 0 && !pools) || (p.cap_recv > 0 && !bank_rows)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!topk_idx || !z || !pool_slot || !recv_slot)) return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.dispatch_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  return run_dispatch(cfg, p, topk_idx, z, pools, pool_slot, recv_slot, bank_rows, pool_count,
                      expert_count, counts, ws, static_cast<hipStream_t>(stream), nullptr);
}

// ---- dispatch without allocation -----------------------------------------
// The scratch of moe_dispatch_noalloc (per-wave counters and per-chunk key
// counts, the same bytes moe_dispatch takes as its workspace) lives in this
// file-scope device array: every GPU the library runs on holds one copy at
// its own address until the process ends.  In host code the array's name is
// a host-side stand-in, never a device address: only the pointer that
// hipGetSymbolAddress returns for the current device is handed to kernels.
namespace {

constexpr int64_t kNoallocScratchBytes = int64_t(4) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char noalloc_scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the array, looked up once per device (with
// that device current) on the first call that runs there.
moe_status noalloc_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

MOE_API int64_t moe_dispatch_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

MOE_API moe_status moe_dispatch_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* z,
                                        void* pools, int32_t* pool_slot, int32_t* recv_slot,
                                        int32_t* bank_rows, int32_t* pool_count, int32_t* expert_count,
                                        int64_t* counts, void* stream) {
  moe_plan p;
  moe_status st = plan_impl(cfg, &p);
  if (st != MOE_OK) return st;
  if (!pool_count || !expert_count || !counts) return MOE_ERR_INVALID_ARG;
  if ((p.pools_bytes > 0 && !pools) || (p.cap_recv > 0 && !bank_rows)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!topk_idx || !z || !pool_slot || !recv_slot)) return MOE_ERR_INVALID_ARG;
  if (p.dispatch_ws_bytes > kNoallocScratchBytes) return MOE_ERR_WORKSPACE;
  void* scratch = nullptr;
  st = noalloc_scratch_ptr(&scratch);
  if (st != MOE_OK) return st;
  // the kernels clear what they accumulate into (the first workgroup of the
  // count pass zeroes the per-wave counters; every chunk count that is read
  // is written first), so the array's previous contents do not matter
  return run_dispatch(cfg, p, topk_idx, z, pools, pool_slot, recv_slot, bank_rows, pool_count,
                      expert_count, counts, scratch, static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_experts(const moe_config* cfg, const void* pools, const int32_t* bank_rows,
                               const int32_t* expert_count, const void* w_gate, const void* w_up,
                               const void* w_down, void* expert_out, void* ws, size_t ws_bytes,
                               void* stream) {
  moe_plan p;
  moe_status st = plan_impl(cfg, &p);
  if (st != MOE_OK) return st;
  if (!expert_count || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if ((p.pools_bytes > 0 && (!pools || !expert_out)) || (p.cap_recv > 0 && !bank_rows))
    return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.experts_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  return run_experts(cfg, p, pools, bank_rows, expert_count, w_gate, w_up, w_down, expert_out, ws,
                     static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_combine(const moe_config* cfg, const void* expert_out,
                               const int32_t* topk_idx, const int32_t* pool_slot,
                               const int32_t* recv_slot, const float* gates, void* y_latent,
                               void* stream) {
  moe_plan p;
  moe_status st = plan_impl(cfg, &p);
  if (st != MOE_OK) return st;
  // pool-shaped buffers are empty when the sender capacity is 0: then they may be null
  if (cfg->T > 0 && ((p.expert_out_bytes > 0 && !expert_out) || !topk_idx || !pool_slot || !recv_slot || !gates ||
                     !y_latent))
    return MOE_ERR_INVALID_ARG;
  return run_combine(cfg, p, expert_out, topk_idx, pool_slot, recv_slot, gates, y_latent,
                     static_cast<hipStream_t>(stream));
}

namespace {

moe_status forward_impl(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                        const moe_taps* taps, int64_t* counts, void* ws, size_t ws_bytes,
                        void* stream, void* const* events, int n_events) {
  moe_plan p;
  moe_status st = plan_impl(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->top_k > cfg->n_experts) return MOE_ERR_INVALID_ARG;
  // the router GEMM writes fp32 logit rows in 16-byte chunks
  if (cfg->n_experts % 4) return MOE_ERR_UNSUPPORTED;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (!w->w_latent || !w->w_router || !w->w_gate || !w->w_up || !w->w_down || !w->w_up_proj)
    return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.forward_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;

  const moe_taps none{};
  const moe_taps& tp = taps ? *taps : none;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = cfg->T, W = cfg->n_waves, E = cfg->n_experts, P = cfg->n_pools,
                k = cfg->top_k;
  const int64_t L = cfg->d_latent, D = cfg->d_model, S = cfg->n_shared, Fs = cfg->d_ff_shared;
  const int64_t eb = p.elem_bytes;
  const int dt = cfg->dtype;

  Carver cv{static_cast<char*>(ws), 0};
  auto pick = [&](void* tap, int64_t bytes) {
    void* q = cv.take(bytes);
    return tap ? tap : q;
  };
  void* z = pick(tp.z, T * L * eb);
  float* logits = static_cast<float*>(pick(tp.logits, T * E * 4));
  int32_t* topk = static_cast<int32_t*>(pick(tp.topk_idx, T * k * 4));
  float* gates = static_cast<float*>(pick(tp.gates, T * k * 4));
  int32_t* pool_slot = static_cast<int32_t*>(pick(tp.pool_slot, T * k * 4));
  int32_t* recv_slot = static_cast<int32_t*>(pick(tp.recv_slot, T * k * 4));
  int32_t* pool_count = static_cast<int32_t*>(pick(tp.pool_count, W * P * 4));
  int32_t* expert_count = static_cast<int32_t*>(pick(tp.expert_count, W * E * 4));
  int32_t* bank_rows = static_cast<int32_t*>(pick(tp.bank_rows, W * E * p.cap_recv * 4));
  void* pools = pick(tp.pools, p.pools_bytes);
  void* expert_out = pick(tp.expert_out, p.expert_out_bytes);
  void* y_lat = pick(tp.y_latent, T * L * eb);
  void* hs = cv.take(T * S * Fs * eb);
  // Without a y_latent tap, y_lat and the shared hidden rows are the two
  // column blocks of one [T][L + S*Fs] buffer (it fits in the two carves
  // above), so the output projection reads one A operand over all its K
  // ranges.
  int64_t ylat_ld = L, hs_ld = S * Fs;
  if (!tp.y_latent && S > 0 && T * (L + S * Fs) * eb < (int64_t(1) << 32)) {
    hs = static_cast<char*>(y_lat) + L * eb;
    ylat_ld = hs_ld = L + S * Fs;
  }
  int64_t* cnt = static_cast<int64_t*>(pick(counts, 3 * 8));
  void* dws = cv.take(p.dispatch_ws_bytes);
  void* xws = cv.take(p.experts_ws_bytes);

  Marks mk{events, n_events, 0};
  Marks* m = &mk;
  hipError_t e = m->mark(s);  // start of stage 0
  if (e != hipSuccess) return MOE_ERR_HIP;
  // latent projection z = x W_lat^T
  moe::GemmDense g{};
  g.nseg = 1;
  g.seg[0] = {x, D, w->w_latent, D, (int)D};
  g.C = z;
  g.ldc = L;
  g.M = (int)T;
  g.N = (int)L;
  e = moe::launch_gemm_dense(dt, dt, g, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // router logits (fp32) = z W_r^T
  g.seg[0] = {z, L, w->w_router, L, (int)L};
  g.C = logits;
  g.ldc = E;
  g.N = (int)E;
  e = moe::launch_gemm_dense(dt, moe::DT_F32, g, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_topk_gates(logits, w->router_bias, T, (int)E, (int)k, topk, gates, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  st = run_dispatch(cfg, p, topk, z, pools, pool_slot, recv_slot, bank_rows, pool_count,
                    expert_count, cnt, dws, s, m);
  if (st != MOE_OK) return st;
  st = run_experts(cfg, p, pools, bank_rows, expert_count, w->w_gate, w->w_up, w->w_down,
                   expert_out, xws, s, m);
  if (st != MOE_OK) return st;
  st = run_combine(cfg, p, expert_out, topk, pool_slot, recv_slot, gates, y_lat, s, ylat_ld * eb);
  if (st == MOE_OK && m->mark(s) != hipSuccess) st = MOE_ERR_HIP;
  if (st != MOE_OK) return st;
  // shared experts' hidden rows: silu(x Wg_s^T) * (x Wu_s^T), [T][S*Fs]
  if (S > 0) {
    e = moe::launch_swiglu_dense(dt, x, D, w->ws_gate, w->ws_up, (int)S, (int)Fs, (int)D, (int)T,
                                 hs, hs_ld, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (m->mark(s) != hipSuccess) return MOE_ERR_HIP;
  // y = y_lat W_up^T + sum_s hs_s Wd_s^T: one accumulation over K segments
  moe::GemmDense o{};
  o.nseg = 1 + (int)S;
  o.seg[0] = {y_lat, ylat_ld, w->w_up_proj, L, (int)L};
  for (int sh = 0; sh < S; ++sh)
    o.seg[1 + sh] = {static_cast<const char*>(hs) + sh * Fs * eb, hs_ld,
                     static_cast<const char*>(w->ws_down) + sh * D * Fs * eb, Fs, (int)Fs};
  o.C = y;
  o.ldc = D;
  o.M = (int)T;
  o.N = (int)D;
  e = moe::launch_gemm_dense(dt, dt, o, s);
  if (e == hipSuccess) e = m->mark(s);
  return hip_status(e);
}

}  // namespace

MOE_API moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                               const moe_taps* taps, int64_t* counts, void* ws, size_t ws_bytes,
                               void* stream) {
  return forward_impl(cfg, w, x, y, taps, counts, ws, ws_bytes, stream, nullptr, 0);
}

MOE_API moe_status moe_forward_profiled(const moe_config* cfg, const moe_weights* w, const void* x,
                                        void* y, const moe_taps* taps, int64_t* counts, void* ws,
                                        size_t ws_bytes, void* stream, void* const* stage_events,
                                        int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !stage_events)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, x, y, taps, counts, ws, ws_bytes, stream, stage_events, n_events);
}

MOE_API int32_t moe_forward_stage_count(void) { return kStages; }

// ------------------------------------------------------------------ dropless
namespace {

constexpr int kDroplessStages = 11;

moe_status check_dropless(const moe_config* cfg, moe_plan* p) {
  moe_status st = plan_impl(cfg, p);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status run_dispatch_dropless(const moe_config* c, const moe_plan& p, const int32_t* topk, const void* z,
                                 void* xs, int32_t* row_of, int32_t* offsets, int64_t* counts, void* ws,
                                 hipStream_t s, Marks* m) {
  const int64_t n = p.dropless_rows;
  const int64_t nblk = moe::ragged_sort_blocks(n);
  Carver cv{static_cast<char*>(ws), 0};
  int32_t* hist = static_cast<int32_t*>(cv.take(nblk * c->n_experts * 4));
  int32_t* base = static_cast<int32_t*>(cv.take(nblk * c->n_experts * 4));
  hipError_t e = moe::launch_ragged_sort(topk, n, c->n_experts, hist, base, offsets, row_of, counts, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e == hipSuccess) e = moe::launch_ragged_scatter(z, row_of, c->T, c->top_k, p.row_bytes, xs, s);
  if (e == hipSuccess && m) e = m->mark(s);
  return hip_status(e);
}

moe_status run_experts_dropless(const moe_config* c, const moe_plan& p, const void* xs,
                                const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                                void* out, void* ws, hipStream_t s, Marks* m) {
  int64_t ent0, ent1;
  dropless_entries(c, &ent0, &ent1);
  const int64_t n = p.dropless_rows;
  Carver cv{static_cast<char*>(ws), 0};
  int32_t* list0 = static_cast<int32_t*>(cv.take(ent0 * 12));
  int32_t* list1 = static_cast<int32_t*>(cv.take(ent1 * 12));
  int32_t* ntiles = static_cast<int32_t*>(cv.take(8));
  char* H = static_cast<char*>(cv.take(n * c->d_ff * p.elem_bytes));
  const int tn0 = (int)ceil_div(c->d_ff, moe::ragged_gate_up_cols());
  const int tn1 = (int)ceil_div(c->d_latent, moe::ragged_down_cols());
  hipError_t e = moe::launch_ragged_tiles(offsets, c->n_experts, moe::ragged_tile_rows(tall_tiles(c)), tn0, tn1,
                                          list0, list1, ntiles, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::RaggedGemm g{};
  g.A = static_cast<const char*>(xs);
  g.a_row_bytes = p.row_bytes;
  g.offsets = offsets;
  g.list = list0;
  g.ntiles = ntiles;
  g.W0 = static_cast<const char*>(wg);
  g.W1 = static_cast<const char*>(wu);
  g.E = c->n_experts;
  g.F = c->d_ff;
  g.K = c->d_latent;
  g.N = 0;
  g.C = H;
  g.c_row_bytes = (int64_t)c->d_ff * p.elem_bytes;
  e = moe::launch_ragged_gate_up_bf16(g, ent0, tall_tiles(c), s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::RaggedGemm d{};
  d.A = H;
  d.a_row_bytes = (int64_t)c->d_ff * p.elem_bytes;
  d.offsets = offsets;
  d.list = list1;
  d.ntiles = ntiles + 1;
  d.W0 = static_cast<const char*>(wd);
  d.W1 = nullptr;
  d.E = c->n_experts;
  d.F = 0;
  d.K = c->d_ff;
  d.N = c->d_latent;
  d.C = static_cast<char*>(out);
  d.c_row_bytes = p.row_bytes;
  e = moe::launch_ragged_down_bf16(d, ent1, tall_tiles(c), s);
  if (e == hipSuccess && m) e = m->mark(s);
  return hip_status(e);
}

moe_status forward_dropless_impl(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                                 const moe_dropless_taps* taps, int64_t* counts, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events, int n_events) {
  moe_plan p;
  moe_status st = check_dropless(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->top_k > cfg->n_experts) return MOE_ERR_INVALID_ARG;
  if (cfg->n_experts % 4) return MOE_ERR_UNSUPPORTED;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (!w->w_latent || !w->w_router || !w->w_gate || !w->w_up || !w->w_down || !w->w_up_proj)
    return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.dropless_forward_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;

  const moe_dropless_taps none{};
  const moe_dropless_taps& tp = taps ? *taps : none;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = cfg->T, E = cfg->n_experts, k = cfg->top_k;
  const int64_t L = cfg->d_latent, D = cfg->d_model, S = cfg->n_shared, Fs = cfg->d_ff_shared;
  const int64_t eb = p.elem_bytes, n = p.dropless_rows;
  const int dt = cfg->dtype;

  Carver cv{static_cast<char*>(ws), 0};
  auto pick = [&](void* tap, int64_t bytes) {
    void* q = cv.take(bytes);
    return tap ? tap : q;
  };
  void* z = pick(tp.z, T * L * eb);
  float* logits = static_cast<float*>(pick(tp.logits, T * E * 4));
  int32_t* topk = static_cast<int32_t*>(pick(tp.topk_idx, T * k * 4));
  float* gates = static_cast<float*>(pick(tp.gates, T * k * 4));
  int32_t* row_of = static_cast<int32_t*>(pick(tp.row_of, T * k * 4));
  int32_t* offsets = static_cast<int32_t*>(pick(tp.expert_offsets, (E + 1) * 4));
  void* xs = pick(tp.xs, n * L * eb);
  void* out = pick(tp.expert_out, n * L * eb);
  void* y_lat = pick(tp.y_latent, T * L * eb);
  void* hs = cv.take(T * S * Fs * eb);
  // Without a y_latent tap, y_lat and the shared hidden rows are the two
  // column blocks of one [T][L + S*Fs] buffer (it fits in the two carves
  // above), so the output projection reads one A operand over all its K
  // ranges.
  int64_t ylat_ld = L, hs_ld = S * Fs;
  if (!tp.y_latent && S > 0 && T * (L + S * Fs) * eb < (int64_t(1) << 32)) {
    hs = static_cast<char*>(y_lat) + L * eb;
    ylat_ld = hs_ld = L + S * Fs;
  }
  int64_t* cnt = static_cast<int64_t*>(pick(counts, 3 * 8));
  void* dws = cv.take(p.dropless_dispatch_ws_bytes);
  void* xws = cv.take(p.dropless_experts_ws_bytes);

  Marks mk{events, n_events, 0};
  Marks* m = &mk;
  hipError_t e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::GemmDense g{};
  g.nseg = 1;
  g.seg[0] = {x, D, w->w_latent, D, (int)D};
  g.C = z;
  g.ldc = L;
  g.M = (int)T;
  g.N = (int)L;
  e = moe::launch_gemm_dense(dt, dt, g, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  g.seg[0] = {z, L, w->w_router, L, (int)L};
  g.C = logits;
  g.ldc = E;
  g.N = (int)E;
  e = moe::launch_gemm_dense(dt, moe::DT_F32, g, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_topk_gates(logits, w->router_bias, T, (int)E, (int)k, topk, gates, s);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  st = run_dispatch_dropless(cfg, p, topk, z, xs, row_of, offsets, cnt, dws, s, m);
  if (st != MOE_OK) return st;
  st = run_experts_dropless(cfg, p, xs, offsets, w->w_gate, w->w_up, w->w_down, out, xws, s, m);
  if (st != MOE_OK) return st;
  e = moe::launch_ragged_combine(dt, out, row_of, gates, T, (int)k, p.row_bytes, y_lat, s, ylat_ld * eb);
  if (e == hipSuccess) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (S > 0) {
    e = moe::launch_swiglu_dense(dt, x, D, w->ws_gate, w->ws_up, (int)S, (int)Fs, (int)D, (int)T, hs, hs_ld,
                                 s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (m->mark(s) != hipSuccess) return MOE_ERR_HIP;
  moe::GemmDense o{};
  o.nseg = 1 + (int)S;
  o.seg[0] = {y_lat, ylat_ld, w->w_up_proj, L, (int)L};
  for (int sh = 0; sh < S; ++sh)
    o.seg[1 + sh] = {static_cast<const char*>(hs) + sh * Fs * eb, hs_ld,
                     static_cast<const char*>(w->ws_down) + sh * D * Fs * eb, Fs, (int)Fs};
  o.C = y;
  o.ldc = D;
  o.M = (int)T;
  o.N = (int)D;
  e = moe::launch_gemm_dense(dt, dt, o, s);
  if (e == hipSuccess) e = m->mark(s);
  return hip_status(e);
}

}  // namespace

MOE_API moe_status moe_dispatch_dropless(const moe_config* cfg, const int32_t* topk_idx, const void* z,
                                         void* xs, int32_t* row_of, int32_t* expert_offsets,
                                         int64_t* counts, void* ws, size_t ws_bytes, void* stream) {
  moe_plan p;
  moe_status st = check_dropless(cfg, &p);
  if (st != MOE_OK) return st;
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!topk_idx || !z || !xs || !row_of)) return MOE_ERR_INVALID_ARG;
  if (p.dropless_dispatch_ws_bytes > 0 &&
      (!ws || (int64_t)ws_bytes < p.dropless_dispatch_ws_bytes || !aligned256(ws)))
    return MOE_ERR_WORKSPACE;
  return run_dispatch_dropless(cfg, p, topk_idx, z, xs, row_of, expert_offsets, counts, ws,
                               static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_experts_dropless(const moe_config* cfg, const void* xs, const int32_t* expert_offsets,
                                        const void* w_gate, const void* w_up, const void* w_down,
                                        void* expert_out, void* ws, size_t ws_bytes, void* stream) {
  moe_plan p;
  moe_status st = check_dropless(cfg, &p);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!xs || !expert_out)) return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.dropless_experts_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  return run_experts_dropless(cfg, p, xs, expert_offsets, w_gate, w_up, w_down, expert_out, ws,
                              static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_combine_dropless(const moe_config* cfg, const void* expert_out, const int32_t* row_of,
                                        const float* gates, void* y_latent, void* stream) {
  moe_plan p;
  moe_status st = check_dropless(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!expert_out || !row_of || !gates || !y_latent)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_ragged_combine(cfg->dtype, expert_out, row_of, gates, cfg->T, cfg->top_k,
                                               p.row_bytes, y_latent, static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_forward_dropless(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                                        const moe_dropless_taps* taps, int64_t* counts, void* ws,
                                        size_t ws_bytes, void* stream) {
  return forward_dropless_impl(cfg, w, x, y, taps, counts, ws, ws_bytes, stream, nullptr, 0);
}

MOE_API int32_t moe_forward_dropless_stage_count(void) { return kDroplessStages; }

MOE_API moe_status moe_forward_dropless_profiled(const moe_config* cfg, const moe_weights* w, const void* x,
                                                 void* y, const moe_dropless_taps* taps, int64_t* counts,
                                                 void* ws, size_t ws_bytes, void* stream,
                                                 void* const* stage_events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !stage_events)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  return forward_dropless_impl(cfg, w, x, y, taps, counts, ws, ws_bytes, stream, stage_events, n_events);
}

// ------------------------------------------------------------------ backward
namespace {

constexpr int kBackwardStages = 11;

moe_status check_backward(const moe_config* cfg, moe_plan* p) {
  moe_status st = plan_impl(cfg, p);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16 || cfg->d_latent % 256 || cfg->d_ff % 256) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status run_combine_bwd(const moe_config* c, const moe_plan& p, const void* expert_out, const int32_t* topk,
                           const int32_t* pool_slot, const int32_t* recv_slot, const float* gates,
                           const void* dy, float* d_gates, void* d_expert_out, hipStream_t s) {
  moe::CombineBwdArgs a{};
  a.expert_out = expert_out;
  a.dy = dy;
  a.topk = topk;
  a.pool_slot = pool_slot;
  a.recv_slot = recv_slot;
  a.gates = gates;
  a.T = c->T;
  a.Tw = p.tokens_per_wave;
  a.k = c->top_k;
  a.E = c->n_experts;
  a.P = c->n_pools;
  a.cap_send = p.cap_send;
  a.row_bytes = p.row_bytes;
  a.d_gates = d_gates;
  a.d_expert_out = d_expert_out;
  return hip_status(moe::launch_combine_bwd(a, s));
}

// Where the experts' backward finds its rows: the capped path's pools and
// bank lists, or the dropless variant's expert-ordered buffers.
struct BwdRows {
  const int32_t* bank_rows;       // capped
  const int32_t* expert_count;
  const int32_t* expert_offsets;  // dropless (non-NULL selects it)
  const void* u;                  // pools, or xs
  const void* d_out;              // d_expert_out
  void* d_in;                     // du out: d_pool_rows, or d_xs
};

moe_status run_experts_bwd(const moe_config* c, const moe_plan& p, const BwdRows& src, const void* wg, const void* wu,
                           const void* wd, void* dwg, void* dwu, void* dwd, void* ws, hipStream_t s, Marks* m) {
  const int E = c->n_experts;
  const bool ragged = src.expert_offsets != nullptr;
  const int64_t L = c->d_latent, F = c->d_ff, R = ragged ? p.dropless_backward_rows : p.backward_rows;
  int64_t epre, edh, edu;
  backward_entries(c, R, &epre, &edh, &edu);
  Carver cv{static_cast<char*>(ws), 0};
  int32_t* counts = static_cast<int32_t*>(cv.take(E * 4));
  int32_t* offsets = static_cast<int32_t*>(cv.take((int64_t)(E + 1) * 4));
  int32_t* gidx = static_cast<int32_t*>(cv.take(R * 4));
  int32_t* list_pre = static_cast<int32_t*>(cv.take(epre * 12));
  int32_t* list_dh = static_cast<int32_t*>(cv.take(edh * 12));
  int32_t* list_du = static_cast<int32_t*>(cv.take(edu * 12));
  int32_t* ntiles = static_cast<int32_t*>(cv.take(16));
  char* U = static_cast<char*>(cv.take(R * L * 2));
  char* DO = static_cast<char*>(cv.take(R * L * 2));
  char* DH = static_cast<char*>(cv.take(R * F * 2));
  char* DADB = static_cast<char*>(cv.take(R * 2 * F * 2));
  char* H = static_cast<char*>(cv.take(R * F * 2));
  // one M-tile structure serves the recompute (expert tile) and dh (dgrad
  // tile) lists, so the two tiles must have the same row count
  const int bm = moe::bwd_dgrad_rows();
  if (bm != moe::ragged_tile_rows(false)) return MOE_ERR_UNSUPPORTED;
  hipError_t e = ragged ? moe::launch_bwd_layout_ragged(src.expert_offsets, E, p.dropless_rows, counts, offsets,
                                                         gidx, s)
                        : moe::launch_bwd_layout(src.bank_rows, src.expert_count, E, c->n_pools, c->n_waves,
                                                 p.cap_send, p.cap_recv, counts, offsets, gidx, s);
  if (e == hipSuccess)
    e = moe::launch_ragged_tiles(offsets, E, bm, (int)ceil_div(F, moe::ragged_gate_up_cols()),
                                 (int)ceil_div(F, moe::bwd_dgrad_cols()), list_pre, list_dh, ntiles, s);
  if (e == hipSuccess)
    e = moe::launch_ragged_tiles(offsets, E, bm, (int)ceil_div(L, moe::bwd_dgrad_cols()), 0, list_du, list_du,
                                 ntiles + 2, s);
  if (e == hipSuccess && m) e = m->mark(s);
  // u and do rows in the padded expert-major order (zero padding rows)
  const int one_block = 0x7fffffff;  // the dropless buffers are one block of rows
  if (e == hipSuccess)
    e = ragged ? moe::launch_gather_rows(src.u, one_block, 0, p.row_bytes, gidx, offsets + E, R, U, s)
               : moe::launch_gather_rows(src.u, (int)p.cap_send, p.pool_block_bytes, p.row_bytes, gidx, offsets + E,
                                         R, U, s);
  if (e == hipSuccess)
    e = ragged ? moe::launch_gather_rows(src.d_out, one_block, 0, p.row_bytes, gidx, offsets + E, R, DO, s)
               : moe::launch_gather_rows(src.d_out, (int)p.cap_send, p.cap_send * p.row_bytes, p.row_bytes, gidx,
                                         offsets + E, R, DO, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // dh = do W_d
  moe::BwdDgrad d{};
  d.A = DO;
  d.a_row_bytes = L * 2;
  d.offsets = offsets;
  d.counts = counts;
  d.list = list_dh;
  d.ntiles = ntiles + 1;
  d.W0 = static_cast<const char*>(wd);
  d.E = E;
  d.K = (int)L;
  d.N = (int)F;
  d.F = (int)F;
  d.C = DH;
  d.c_row_bytes = F * 2;
  e = moe::launch_bwd_dh(d, edh, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // recompute a = u W_g^T, b = u W_u^T; SwiGLU backward: da, db, h
  moe::RaggedGemm g{};
  g.A = U;
  g.a_row_bytes = L * 2;
  g.offsets = offsets;
  g.list = list_pre;
  g.ntiles = ntiles;
  g.W0 = static_cast<const char*>(wg);
  g.W1 = static_cast<const char*>(wu);
  g.E = E;
  g.F = (int)F;
  g.K = (int)L;
  g.C = DADB;
  g.c_row_bytes = 2 * F * 2;
  g.dH = DH;
  g.dh_row_bytes = F * 2;
  g.H = H;
  g.h_row_bytes = F * 2;
  e = moe::launch_ragged_swiglu_bwd_bf16(g, epre, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // du = da W_g + db W_u, rows back to their pool slots
  moe::BwdDgrad u{};
  u.A = DADB;
  u.a_row_bytes = 2 * F * 2;
  u.a_seg_bytes = F * 2;
  u.offsets = offsets;
  u.counts = counts;
  u.list = list_du;
  u.ntiles = ntiles + 2;
  u.W0 = static_cast<const char*>(wg);
  u.W1 = static_cast<const char*>(wu);
  u.E = E;
  u.K = (int)F;
  u.N = (int)L;
  u.F = (int)F;
  u.C = static_cast<char*>(src.d_in);
  u.c_row_bytes = p.row_bytes;
  u.c_index = gidx;
  e = moe::launch_bwd_du(u, edu, s);
  if (e == hipSuccess && m) e = m->mark(s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // weight gradients over each expert's padded rows
  const int tile = moe::bwd_wgrad_tile();
  auto wgrad = [&](const char* X, int64_t xr, int64_t xc, const char* Y, int64_t yr, int M, int N, void* C) {
    moe::BwdWgrad w{};
    w.X = X;
    w.x_row_bytes = xr;
    w.x_col_bytes = xc;
    w.Y = Y;
    w.y_row_bytes = yr;
    w.y_col_bytes = 0;
    w.offsets = offsets;
    w.counts = counts;
    w.E = E;
    w.M = M;
    w.N = N;
    w.tiles_m = M / tile;
    w.tiles_n = N / tile;
    w.C = static_cast<char*>(C);
    hipError_t r = moe::launch_bwd_wgrad(w, s);
    if (r == hipSuccess && m) r = m->mark(s);
    return r;
  };
  e = wgrad(DO, L * 2, 0, H, F * 2, (int)L, (int)F, dwd);
  if (e == hipSuccess) e = wgrad(DADB, 2 * F * 2, 0, U, L * 2, (int)F, (int)L, dwg);
  if (e == hipSuccess) e = wgrad(DADB, 2 * F * 2, F * 2, U, L * 2, (int)F, (int)L, dwu);
  return hip_status(e);
}

moe_status run_dispatch_bwd(const moe_config* c, const moe_plan& p, const int32_t* topk, const int32_t* pool_slot,
                            const int32_t* recv_slot, const void* d_pool_rows, void* dz, hipStream_t s) {
  return run_combine(c, p, d_pool_rows, topk, pool_slot, recv_slot, nullptr, dz, s);
}

moe_status backward_impl(const moe_config* cfg, const moe_weights* w, const moe_taps* sv, const void* dy,
                         void* dz, float* d_logits, void* dwg, void* dwu, void* dwd, void* ws, size_t ws_bytes,
                         void* stream, void* const* events, int n_events) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (!w || !sv || !w->w_gate || !w->w_up || !w->w_down || !dwg || !dwu || !dwd || !sv->expert_count)
    return MOE_ERR_INVALID_ARG;
  // pool-shaped buffers are empty when a capacity is 0: then they may be null
  if ((p.pools_bytes > 0 && (!sv->pools || !sv->expert_out)) || (p.cap_recv > 0 && !sv->bank_rows))
    return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!sv->topk_idx || !sv->gates || !sv->pool_slot || !sv->recv_slot || !dy || !dz || !d_logits))
    return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.backward_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Marks marks{events, n_events, 0};
  Marks* m = events ? &marks : nullptr;
  Carver cv{static_cast<char*>(ws), 0};
  const int64_t T = cfg->T, k = cfg->top_k;
  float* d_gates = static_cast<float*>(cv.take(T * k * 4));
  void* d_expert_out = cv.take(p.expert_out_bytes);
  void* d_pool_rows = cv.take(p.expert_out_bytes);
  void* ews = cv.take(p.experts_bwd_ws_bytes);
  hipError_t e = m ? m->mark(s) : hipSuccess;
  if (e != hipSuccess) return MOE_ERR_HIP;
  st = run_combine_bwd(cfg, p, sv->expert_out, sv->topk_idx, sv->pool_slot, sv->recv_slot, sv->gates, dy, d_gates,
                       d_expert_out, s);
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  if (st == MOE_OK) {
    const BwdRows src{sv->bank_rows, sv->expert_count, nullptr, sv->pools, d_expert_out, d_pool_rows};
    st = run_experts_bwd(cfg, p, src, w->w_gate, w->w_up, w->w_down, dwg, dwu, dwd, ews, s, m);
  }
  if (st == MOE_OK)
    st = run_dispatch_bwd(cfg, p, sv->topk_idx, sv->pool_slot, sv->recv_slot, d_pool_rows, dz, s);
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  if (st == MOE_OK)
    st = hip_status(moe::launch_route_bwd(sv->topk_idx, sv->gates, d_gates, T, (int)k, cfg->n_experts, d_logits, s));
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  return st;
}

}  // namespace

MOE_API moe_status moe_combine_backward(const moe_config* cfg, const void* expert_out, const int32_t* topk_idx,
                                        const int32_t* pool_slot, const int32_t* recv_slot, const float* gates,
                                        const void* dy_latent, float* d_gates, void* d_expert_out, void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && ((p.expert_out_bytes > 0 && (!expert_out || !d_expert_out)) || !topk_idx || !pool_slot ||
                     !recv_slot || !gates || !dy_latent || !d_gates))
    return MOE_ERR_INVALID_ARG;
  return run_combine_bwd(cfg, p, expert_out, topk_idx, pool_slot, recv_slot, gates, dy_latent, d_gates,
                         d_expert_out, static_cast<hipStream_t>(stream));
}

MOE_API moe_status moe_experts_backward(const moe_config* cfg, const void* pools, const int32_t* bank_rows,
                                        const int32_t* expert_count, const void* w_gate, const void* w_up,
                                        const void* w_down, const void* d_expert_out, void* d_pool_rows,
                                        void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                        void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (!expert_count || !w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down) return MOE_ERR_INVALID_ARG;
  if ((p.pools_bytes > 0 && (!pools || !d_expert_out || !d_pool_rows)) || (p.cap_recv > 0 && !bank_rows))
    return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.experts_bwd_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  const BwdRows src{bank_rows, expert_count, nullptr, pools, d_expert_out, d_pool_rows};
  return run_experts_bwd(cfg, p, src, w_gate, w_up, w_down, dw_gate, dw_up, dw_down, ws,
                         static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_dispatch_backward(const moe_config* cfg, const int32_t* topk_idx, const int32_t* pool_slot,
                                         const int32_t* recv_slot, const void* d_pool_rows, void* dz,
                                         void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!topk_idx || !pool_slot || !recv_slot || (p.expert_out_bytes > 0 && !d_pool_rows) || !dz))
    return MOE_ERR_INVALID_ARG;
  return run_dispatch_bwd(cfg, p, topk_idx, pool_slot, recv_slot, d_pool_rows, dz,
                          static_cast<hipStream_t>(stream));
}

MOE_API moe_status moe_route_backward(const moe_config* cfg, const int32_t* topk_idx, const float* gates,
                                      const float* d_gates, float* d_logits, void* stream) {
  moe_status st = check_route_shape(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!topk_idx || !gates || !d_gates || !d_logits)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_route_bwd(topk_idx, gates, d_gates, cfg->T, cfg->top_k, cfg->n_experts, d_logits,
                                          static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_backward_routed(const moe_config* cfg, const moe_weights* w, const moe_taps* saved,
                                       const void* dy_latent, void* dz, float* d_logits, void* dw_gate,
                                       void* dw_up, void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(cfg, w, saved, dy_latent, dz, d_logits, dw_gate, dw_up, dw_down, ws, ws_bytes, stream,
                       nullptr, 0);
}

MOE_API int32_t moe_backward_routed_stage_count(void) { return kBackwardStages; }

MOE_API moe_status moe_backward_routed_profiled(const moe_config* cfg, const moe_weights* w, const moe_taps* saved,
                                                const void* dy_latent, void* dz, float* d_logits, void* dw_gate,
                                                void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                                void* stream, void* const* stage_events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !stage_events)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  return backward_impl(cfg, w, saved, dy_latent, dz, d_logits, dw_gate, dw_up, dw_down, ws, ws_bytes, stream,
                       stage_events, n_events);
}

// ------------------------------------------------------------------ dropless backward
namespace {

moe_status run_combine_bwd_dropless(const moe_config* c, const moe_plan& p, const void* expert_out,
                                    const int32_t* row_of, const float* gates, const void* dy, float* d_gates,
                                    void* d_expert_out, hipStream_t s) {
  moe::CombineBwdArgs a{};
  a.expert_out = expert_out;
  a.dy = dy;
  a.row_of = row_of;
  a.gates = gates;
  a.T = c->T;
  a.Tw = p.tokens_per_wave > 0 ? p.tokens_per_wave : 1;
  a.k = c->top_k;
  a.E = c->n_experts;
  a.P = c->n_pools;
  a.cap_send = p.cap_send;
  a.row_bytes = p.row_bytes;
  a.d_gates = d_gates;
  a.d_expert_out = d_expert_out;
  return hip_status(moe::launch_combine_bwd(a, s));
}

moe_status backward_dropless_impl(const moe_config* cfg, const moe_weights* w, const moe_dropless_taps* sv,
                                  const void* dy, void* dz, float* d_logits, void* dwg, void* dwu, void* dwd,
                                  void* ws, size_t ws_bytes, void* stream, void* const* events, int n_events) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (!w || !sv || !w->w_gate || !w->w_up || !w->w_down || !dwg || !dwu || !dwd || !sv->expert_offsets)
    return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!sv->topk_idx || !sv->gates || !sv->row_of || !sv->xs || !sv->expert_out || !dy || !dz ||
                     !d_logits))
    return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.dropless_backward_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Marks marks{events, n_events, 0};
  Marks* m = events ? &marks : nullptr;
  Carver cv{static_cast<char*>(ws), 0};
  const int64_t T = cfg->T, k = cfg->top_k, n = p.dropless_rows;
  float* d_gates = static_cast<float*>(cv.take(T * k * 4));
  void* d_expert_out = cv.take(n * p.row_bytes);
  void* d_xs = cv.take(n * p.row_bytes);
  void* ews = cv.take(p.dropless_experts_bwd_ws_bytes);
  hipError_t e = m ? m->mark(s) : hipSuccess;
  if (e != hipSuccess) return MOE_ERR_HIP;
  st = run_combine_bwd_dropless(cfg, p, sv->expert_out, sv->row_of, sv->gates, dy, d_gates, d_expert_out, s);
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  if (st == MOE_OK) {
    const BwdRows src{nullptr, nullptr, sv->expert_offsets, sv->xs, d_expert_out, d_xs};
    st = run_experts_bwd(cfg, p, src, w->w_gate, w->w_up, w->w_down, dwg, dwu, dwd, ews, s, m);
  }
  if (st == MOE_OK)
    st = hip_status(moe::launch_ragged_combine(cfg->dtype, d_xs, sv->row_of, nullptr, T, (int)k, p.row_bytes, dz, s));
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  if (st == MOE_OK)
    st = hip_status(moe::launch_route_bwd(sv->topk_idx, sv->gates, d_gates, T, (int)k, cfg->n_experts, d_logits, s));
  if (st == MOE_OK && m) st = hip_status(m->mark(s));
  return st;
}

}  // namespace

MOE_API moe_status moe_combine_backward_dropless(const moe_config* cfg, const void* expert_out,
                                                 const int32_t* row_of, const float* gates, const void* dy_latent,
                                                 float* d_gates, void* d_expert_out, void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!expert_out || !row_of || !gates || !dy_latent || !d_gates || !d_expert_out))
    return MOE_ERR_INVALID_ARG;
  return run_combine_bwd_dropless(cfg, p, expert_out, row_of, gates, dy_latent, d_gates, d_expert_out,
                                  static_cast<hipStream_t>(stream));
}

MOE_API moe_status moe_experts_backward_dropless(const moe_config* cfg, const void* xs, const int32_t* expert_offsets,
                                                 const void* w_gate, const void* w_up, const void* w_down,
                                                 const void* d_expert_out, void* d_xs, void* dw_gate, void* dw_up,
                                                 void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!xs || !d_expert_out || !d_xs)) return MOE_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.dropless_experts_bwd_ws_bytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  const BwdRows src{nullptr, nullptr, expert_offsets, xs, d_expert_out, d_xs};
  return run_experts_bwd(cfg, p, src, w_gate, w_up, w_down, dw_gate, dw_up, dw_down, ws,
                         static_cast<hipStream_t>(stream), nullptr);
}

MOE_API moe_status moe_dispatch_backward_dropless(const moe_config* cfg, const int32_t* row_of, const void* d_xs,
                                                  void* dz, void* stream) {
  moe_plan p;
  moe_status st = check_backward(cfg, &p);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!row_of || !d_xs || !dz)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_ragged_combine(cfg->dtype, d_xs, row_of, nullptr, cfg->T, cfg->top_k, p.row_bytes,
                                               dz, static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_backward_dropless(const moe_config* cfg, const moe_weights* w, const moe_dropless_taps* saved,
                                         const void* dy_latent, void* dz, float* d_logits, void* dw_gate,
                                         void* dw_up, void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  return backward_dropless_impl(cfg, w, saved, dy_latent, dz, d_logits, dw_gate, dw_up, dw_down, ws, ws_bytes,
                                stream, nullptr, 0);
}

MOE_API moe_status moe_backward_dropless_profiled(const moe_config* cfg, const moe_weights* w,
                                                  const moe_dropless_taps* saved, const void* dy_latent, void* dz,
                                                  float* d_logits, void* dw_gate, void* dw_up, void* dw_down,
                                                  void* ws, size_t ws_bytes, void* stream,
                                                  void* const* stage_events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !stage_events)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  return backward_dropless_impl(cfg, w, saved, dy_latent, dz, d_logits, dw_gate, dw_up, dw_down, ws, ws_bytes,
                                stream, stage_events, n_events);
}
