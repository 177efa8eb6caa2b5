// Internal launchers of the gfx950 kernels (host side).  Each launcher
// enqueues on `s` and returns hipGetLastError(); shapes are validated by the
// C-ABI layer before any call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// element types (same values as moe_dtype)
enum Dt : int { DT_F32 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------- GEMMs
// C[M][N] (+)= sum over segments of A_s[M][K_s] * B_s[N][K_s]^T, fp32 accumulate.
struct GemmSeg {
  const void* A;
  int64_t lda;  // elements
  const void* B;
  int64_t ldb;  // elements
  int K;
};
constexpr int kMaxSegs = 4;
struct GemmDense {
  GemmSeg seg[kMaxSegs];
  int nseg;
  void* C;
  int64_t ldc;  // elements of the output type
  int M, N;
};
// in_dt: element type of A and B; out_dt: element type of C.
hipError_t launch_gemm_dense(int in_dt, int out_dt, const GemmDense& g, hipStream_t s);

// C[m][g*F + f] = silu(A[m] . Wg[g][f]) * (A[m] . Wu[g][f]) for g < G, f < F
// (the shared experts; Wg, Wu are [G][F][K]).
hipError_t launch_swiglu_dense(int dt, const void* A, int64_t lda, const void* Wg,
                               const void* Wu, int G, int F, int K, int M, void* C,
                               int64_t ldc, hipStream_t s);

// Routed experts, gate/up half: for expert e and its row m < rows_total[e],
// u = pool row erow[e][m] (flat (w*P + p)*C_send + s index), and
// H[e][m][f] = silu(u . Wg[e][f]) * (u . Wu[e][f]).
struct ExpertGateUp {
  const char* pools;
  int64_t block_bytes;
  int64_t row_bytes;
  int cap_send;
  const int32_t* erow;        // [E][max_rows]
  const int32_t* rows_total;  // [E]
  int E, max_rows, F, L;
  const void* Wg;
  const void* Wu;
  void* H;  // [E][max_rows][F]
};
hipError_t launch_expert_gate_up(int dt, const ExpertGateUp& a, hipStream_t s);

// Routed experts, down half: expert_out row erow[e][m] = H[e][m] . Wd[e]^T.
struct ExpertDown {
  const void* H;
  const int32_t* erow;
  const int32_t* rows_total;
  int E, max_rows, F, L;
  const void* Wd;   // [E][L][F]
  void* out;        // [W*P*C_send][L]
};
hipError_t launch_expert_down(int dt, const ExpertDown& a, hipStream_t s);

// bf16 paths on the gfx950 GEMM core (gemm_bf16.hip); the generic dense
// launchers above dispatch to them for bf16 inputs and outputs.
hipError_t launch_gemm_dense_bf16(const GemmDense& g, hipStream_t s);
// bf16 operands, fp32 output on the gfx950 core (the router logits), for
// one K range of whole K tiles and whole 16-byte output chunks.
bool dense_f32out_supported(const GemmDense& g);
hipError_t launch_dense_f32out_bf16(const GemmDense& g, hipStream_t s);
hipError_t launch_swiglu_dense_bf16(const void* A, int64_t lda, const void* Wg, const void* Wu, int G,
                                    int F, int K, int M, void* C, int64_t ldc, hipStream_t s);

// ---------------------------------------------------------------- routing
hipError_t launch_topk_gates(const float* logits, const float* bias, int64_t T, int E,
                             int k, int32_t* topk_idx, float* gates, hipStream_t s);

// Next-step balancing bias from histogram quantiles of the logits (bias.hip).
int bias_max_bins();
int64_t bias_ws_bytes(int64_t T, int E, int nb);
// events: null, or 5 hipEvent_t recorded around the 4 launches
hipError_t launch_bias_update(const float* logits, int64_t T, int E, int k, int nb, float* bias, int32_t* hist_out,
                              float* lohi_out, void* ws, hipStream_t s, void* const* events);

// ---------------------------------------------------------------- dispatch
struct DispatchArgs {
  const int32_t* topk;
  int64_t T;
  int k, E, P, W;
  int64_t Tw, cap_send, cap_recv;
  int32_t* pool_slot;
  int32_t* recv_slot;
  int32_t* pool_count;   // [W][P]
  char* pools;           // block layout
  int64_t block_bytes, ids_offset, row_bytes;
  int64_t* wave_counts;  // [W][3] workspace
  int64_t* counts;       // [3] or null
  int32_t* chunk_counts; // [W][n_chunks][E + P] workspace: per-chunk key counts
  int n_chunks;          // chunks of the slot scan per wave (assign_chunks)
};
// Chunks of the slot scan per wave: ceil(Tw * k / 1024), at least 1.
int assign_chunks(int64_t Tw, int k);
hipError_t launch_assign(const DispatchArgs& a, hipStream_t s);
hipError_t launch_scatter_rows(const DispatchArgs& a, const void* z, hipStream_t s);
hipError_t launch_recv_bin(const DispatchArgs& a, int32_t* bank_rows,
                           int32_t* expert_count, hipStream_t s);
hipError_t launch_expert_rows(const int32_t* bank_rows, const int32_t* expert_count,
                              int E, int P, int W, int64_t cap_send, int64_t cap_recv,
                              int32_t* erow, int32_t* rows_total, int max_rows,
                              hipStream_t s);

// bf16 path: expert-major offsets [E+1] of the kept rows and their flat pool
// row indices gidx [offsets[E]] (the ragged GEMMs then run over them).
hipError_t launch_expert_gidx(const int32_t* bank_rows, const int32_t* expert_count, int E, int P, int W,
                              int64_t cap_send, int64_t cap_recv, int32_t* offsets, int32_t* gidx,
                              hipStream_t s);

// ---------------------------------------------------------------- combine
struct CombineArgs {
  const char* expert_out;
  const int32_t* topk;
  const int32_t* pool_slot;
  const int32_t* recv_slot;
  const float* gates;
  int64_t T, Tw;
  int k, E, P;
  int64_t cap_send, row_bytes;
  void* y;
  int64_t y_pitch;  // bytes between output rows; 0: row_bytes
};
hipError_t launch_combine(int dt, const CombineArgs& a, hipStream_t s);

hipError_t launch_zero_i64(int64_t* p, int n, hipStream_t s);

// ---------------------------------------------------------------- dropless
// Stable counting sort of n assignments by expert (ragged.hip): chunks of
// kRaggedChunk assignments; hist and base are [blocks][E] int32.
constexpr int kRaggedChunk = 4096;
int ragged_sort_blocks(int64_t n);
hipError_t launch_ragged_sort(const int32_t* topk, int64_t n, int E, int32_t* hist, int32_t* base,
                              int32_t* offsets, int32_t* row_of, int64_t* counts, hipStream_t s);
hipError_t launch_ragged_scatter(const void* z, const int32_t* row_of, int64_t T, int k, int64_t row_bytes,
                                 void* xs, hipStream_t s);
// Tile lists of the ragged grouped GEMMs: (expert, n tile, m tile) int32
// triples, M tiles of bm rows; ntiles[0], ntiles[1] = entries of each list.
hipError_t launch_ragged_tiles(const int32_t* offsets, int E, int bm, int tiles_n0, int tiles_n1,
                               int32_t* list0, int32_t* list1, int32_t* ntiles, hipStream_t s);
// y_pitch: bytes between output rows (0: row_bytes)
hipError_t launch_ragged_combine(int dt, const void* out, const int32_t* row_of, const float* gates, int64_t T,
                                 int k, int64_t row_bytes, void* y, hipStream_t s, int64_t y_pitch = 0);

// Ragged grouped GEMMs (bf16, gemm_bf16.hip).  Expert e's rows are rows
// [offsets[e], offsets[e+1]) of A and of C.
struct RaggedGemm {
  const char* A;
  int64_t a_row_bytes;
  // optional gather of A rows: row i of the expert-major order is pool row
  // a_index[i] = block * a_block_rows + slot, at A + block * a_block_bytes +
  // slot * a_row_bytes (NULL: row i at A + i * a_row_bytes)
  const int32_t* a_index;
  int a_block_rows;
  int64_t a_block_bytes;
  // optional scatter of C rows: row i goes to C + c_index[i] * c_row_bytes
  const int32_t* c_index;
  const int32_t* offsets;  // [E+1]
  const int32_t* list;     // tile list of this GEMM
  const int32_t* ntiles;   // device: entries of the list
  const char* W0;          // gate weights [E][F][K], or down weights [E][N][K]
  const char* W1;          // up weights [E][F][K] (SwiGLU only)
  int E, F, K, N;
  char* C;
  int64_t c_row_bytes;
  // the backward's SwiGLU epilogue: dh rows in (bf16), h rows out; C gets
  // [da | db]
  const char* dH;
  int64_t dh_row_bytes;
  char* H;
  int64_t h_row_bytes;
};
// M rows per tile (192, or 256 with `tall`: for experts of thousands of rows)
// and N columns (features for the SwiGLU) per tile, the same for both.
int ragged_tile_rows(bool tall);
int ragged_gate_up_cols();
int ragged_down_cols();
hipError_t launch_ragged_gate_up_bf16(const RaggedGemm& g, int64_t max_entries, bool tall, hipStream_t s);
hipError_t launch_ragged_down_bf16(const RaggedGemm& g, int64_t max_entries, bool tall, hipStream_t s);
// The backward's recompute of the SwiGLU pre-activations a = u W_g^T,
// b = u W_u^T (fp32, never stored) with the SwiGLU backward in the
// epilogue: from dh (g.dH) it writes da | db (g.C) and h (g.H), bf16.
hipError_t launch_ragged_swiglu_bwd_bf16(const RaggedGemm& g, int64_t max_entries, hipStream_t s);

// ---------------------------------------------------------------- backward
// Routed-path backward (bf16).  Row moves and indices (backward.hip):
// counts[e] = rows expert e kept, offsets = the padded expert-major layout
// (every expert rounded up to 64 rows), gidx[i] = flat pool row of padded
// row i or -1 for padding.
hipError_t launch_bwd_layout(const int32_t* bank_rows, const int32_t* expert_count, int E, int P, int W,
                             int64_t cap_send, int64_t cap_recv, int32_t* counts, int32_t* offsets, int32_t* gidx,
                             hipStream_t s);
// The same from the dropless variant's expert offsets over n rows:
// gidx[i] = the row of the expert-ordered buffer, -1 for padding.
hipError_t launch_bwd_layout_ragged(const int32_t* expert_offsets, int E, int64_t n, int32_t* counts,
                                    int32_t* offsets, int32_t* gidx, hipStream_t s);
// dst row i = pool row gidx[i] of src (blocks of block_rows rows) or zeros;
// *nrows rows (device), at most max_rows.
hipError_t launch_gather_rows(const void* src, int block_rows, int64_t block_bytes, int64_t row_bytes,
                              const int32_t* gidx, const int32_t* nrows, int64_t max_rows, void* dst,
                              hipStream_t s);
struct CombineBwdArgs {
  const void* expert_out;  // [W][P][C_send][L], or [T*k][L] with row_of
  const void* dy;          // [T][L]
  const int32_t* row_of;   // dropless: row of each assignment (NULL: pool slots)
  const int32_t* topk;
  const int32_t* pool_slot;
  const int32_t* recv_slot;
  const float* gates;
  int64_t T, Tw;
  int k, E, P;
  int64_t cap_send, row_bytes;
  float* d_gates;       // [T][k]
  void* d_expert_out;   // [W][P][C_send][L], kept rows written
};
hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t s);
hipError_t launch_route_bwd(const int32_t* topk, const float* gates, const float* d_gates, int64_t T, int k, int E,
                            float* d_logits, hipStream_t s);

// Grouped dgrad / wgrad GEMMs (gemm_bwd.hip) over the padded layout.
struct BwdDgrad {
  const char* A;          // padded rows: do (dh) or [da | db] (du)
  int64_t a_row_bytes;
  int64_t a_seg_bytes;    // du: byte offset of db inside an A row
  const int32_t* offsets;  // [E+1] padded
  const int32_t* counts;   // [E]
  const int32_t* list;
  const int32_t* ntiles;
  const char* W0;         // [E][K][N]: W_d (dh) or W_g (du)
  const char* W1;         // du: W_u
  int E, K, N, F;
  // output: row i -> C + i * c_row_bytes (dh, padded rows included), or
  // C + c_index[i] * c_row_bytes (du, kept rows only)
  char* C;
  int64_t c_row_bytes;
  const int32_t* c_index;
};
struct BwdWgrad {
  const char* X;          // K-major rows of the M operand
  int64_t x_row_bytes, x_col_bytes;
  const char* Y;          // K-major rows of the N operand
  int64_t y_row_bytes, y_col_bytes;
  const int32_t* offsets;  // [E+1] padded: expert e's rows sit in [offsets[e], offsets[e+1])
  const int32_t* counts;   // [E] rows of expert e; the rest of its padded range is zeros
  int E, M, N;
  int tiles_m, tiles_n;
  char* C;                // [E][M][N]
};
int bwd_dgrad_rows();
int bwd_dgrad_cols();
int bwd_wgrad_tile();
hipError_t launch_bwd_dh(const BwdDgrad& p, int64_t max_entries, hipStream_t s);
hipError_t launch_bwd_du(const BwdDgrad& p, int64_t max_entries, hipStream_t s);
hipError_t launch_bwd_wgrad(const BwdWgrad& p, hipStream_t s);

}  // namespace moe
