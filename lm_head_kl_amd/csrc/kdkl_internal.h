// Internal interface between the C ABI (kdkl_api.cpp) and the HIP kernels (kdkl_kernels.hip).
// Plain C++ types only; not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kdkl {

// Workgroup tile of every MFMA kernel: 256 rows x 256 columns. The top-K entry plan buckets
// cached ids by the same tile, so both constants are shared with the host code.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kMaxK = 1024;  // cached entries per row
constexpr int kMaxTopK = 1024;  // largest K of the offline top-K producer
constexpr int64_t kMaxTopV = 1 << 22;  // token ids fit in the producer's 22-bit key field
constexpr int kMaxVTiles = 16384;  // plan kernel keeps one LDS counter per vocab tile

enum class Dt : int { F32 = 0, BF16 = 1 };

// Kernel kinds for the optional per-launch timing (kd_timing_* in kdkl.h).
enum Kind : int {
    kKindPlan = 0,
    kKindTeacherProb,
    kKindValidate,
    kKindFwd,
    kKindCombine,
    kKindLossFinal,
    kKindBwdGrad,
    kKindTranspose,
    kKindDh,
    kKindDhReduce,
    kKindDw,
    kKindDenseLogits,
    kKindDenseRows,
    kKindSumRows,
    kKindGradZ,
    kKindTopk,
    kNumKinds
};
// Bracket one launch on stream s with timing events (no-ops unless timing is enabled).
void timing_begin(int kind, hipStream_t s);
void timing_end(int kind, hipStream_t s);

struct Shape {
    int64_t N, d, V, K;
    float T;
    float n_norm;  // resolved: > 0
    Dt act, tlog;
};

// Launchers return hipSuccess or the launch error.  All enqueue on `s`.

// Bucket the cached ids of rows [row0, row1) by (row block of 256, vocab tile of 256).
// off: [n_rb][n_vt + 1] int32 (absolute entry offsets), ent: [n_rb * 256 * K] uint32 packed
// (row in block | col in tile << 8 | k << 16).
hipError_t launch_plan(const int32_t* idx, int64_t row0, int64_t row1, int64_t K, int64_t V,
                       int32_t* off, uint32_t* ent, hipStream_t s);

// p_t[n,k] = softmax(t[n,:]/T)[k] for rows [row0, row1), written to pt[(n-row0)*K + k].
hipError_t launch_teacher_prob(const void* tlog, Dt tdt, int64_t row0, int64_t row1, int64_t K,
                               float T, float* pt, hipStream_t s);

// Check ids: bit 0 = out of range, bit 1 = repeated in a row; ORed into *status (zeroed first).
hipError_t launch_validate(const int32_t* idx, int64_t N, int64_t K, int64_t V, uint32_t* status,
                           hipStream_t s);

// Fused forward over the sh.N rows of H: per (row block, vocab split) partial (max, sum) in
// the log2 domain, and zk at every cached id. With zt not null the logits are also stored
// transposed, z^T [Vp][ldzt] (columns: rows of H), for the paths that keep them.
// tiled_S > 0: H and W are stage-tiled copies (launch_tile_rows) with tiled_S stages per row
// block; 0: row-major [N][d] and [V][d].
hipError_t launch_fwd(const Shape& sh, const void* H, const void* W, const int32_t* plan_off,
                      const uint32_t* plan_ent, int n_vsplit, float2* part, float* zk,
                      float* zt, int64_t ldzt, hipStream_t s, int64_t tiled_S = 0);

// Merge partials into lse, compute KL_n (row_kl) and per-block fp64 partial sums.
hipError_t launch_combine(const Shape& sh, const float2* part, int n_part, const float* zk,
                          const void* tlog, float* lse, float* row_kl, double* blk_sum,
                          int* n_blk_out, hipStream_t s);
int combine_blocks(int64_t N);

// loss[0] = T^2/n_norm * sum(blk_sum[0..n_blk)) in a fixed order.
hipError_t launch_loss_final(const Shape& sh, const double* blk_sum, int n_blk, float* loss,
                             hipStream_t s);

// Backward, one chunk of rows [c0, c0 + cc):
//   G_c = g*T/n_norm*(softmax(z/T) - P_t) in the act dtype (entries v >= V zero), rows = the
//   chunk's tokens, K = vocabulary: stage-tiled (g_tiled; row blocks of 256, Vp/SW stages) or
//   K-blocked [Vp/256][cc][256] (entry (t, v) at ((v/256)*cc + t)*256 + v%256);
//   if GT is not null, G_c^T stage-tiled (row blocks of 256, ldgt/SW stages), the chunk's tokens
//   at K columns gt_col0 + [0, cc), zero for [cc, round_up(cc, 32)); ldgt and gt_col0 multiples
//   of 32.
// H and W as in launch_fwd (a stage-tiled H holds the chunk's cc rows alone: row 0 = row c0);
// stage-tiled H and W need a stage-tiled G_c.
hipError_t launch_bwd_grad(const Shape& sh, const void* H, const void* W, const float* lse,
                           const float* pt, const float* grad_loss, int64_t c0, int64_t cc,
                           const int32_t* plan_off, const uint32_t* plan_ent, void* Gc, bool g_tiled,
                           void* GT, int64_t ldgt, int64_t gt_col0, hipStream_t s, int64_t tiled_S = 0);

// The same stage-tiled G_c and G_c^T as launch_bwd_grad, from stored logits z^T [Vp][ldzt]
// (chunk row r in column zt_col0 + r) instead of recomputing them.
hipError_t launch_grad_z(const Shape& sh, const float* zt, int64_t ldzt, int64_t zt_col0,
                         const float* lse, const float* pt, const float* grad_loss, int64_t c0,
                         int64_t cc, const int32_t* plan_off, const uint32_t* plan_ent, void* Gc,
                         void* GT, int64_t ldgt, int64_t gt_col0, hipStream_t s);

// Offline cache: per row of X [N][ld] (V entries), the K largest values and their ids, largest
// first, ties in lower-id order.
hipError_t launch_topk(Dt dt, const void* X, int64_t ld, int64_t N, int64_t V, int64_t K, int32_t* idx,
                       void* val, hipStream_t s);

// Stage-tiled copy of a row-major src [rows][ld] (cols used; cols and ld multiples of 16 bytes):
// blocks of 256 rows x 64 bytes, block (row block b, stage s) at dst + (b*S + s)*16 KB, S =
// tiled_stages(dt, cols), zeros past rows and cols. tiled_bytes gives the size of dst.
int64_t tiled_stages(Dt dt, int64_t cols);
int64_t tiled_bytes(Dt dt, int64_t rows, int64_t cols);
hipError_t launch_tile_rows(Dt dt, const void* src, int64_t ld, int64_t rows, int64_t cols, void* dst,
                            hipStream_t s);

// Transpose of src [rows][lds] (cols used) into a stage-tiled operand with row blocks of 320 and
// kdst K columns (kdst/SW stages): result row c < cols holds src[r][c] at K column k0 + r for r <
// rows, zero for rows <= r < rows_pad. cols, lds and rows_pad multiples of 8; kdst and k0
// multiples of 32. The result takes round_up(cols, 320) * kdst elements. With tiled_copy not
// null, src is also copied as launch_tile_rows would (rows_pad rows, a multiple of 256).
hipError_t launch_transpose(Dt dt, const void* src, int64_t lds, int64_t rows, int64_t cols, void* dst,
                            int64_t kdst, int64_t k0, int64_t rows_pad, hipStream_t s,
                            void* tiled_copy = nullptr);

// dH rows [c0, c0+cc) = G_c W. With WT not null, G_c is the stage-tiled tile written by
// launch_bwd_grad and WT is W^T from launch_transpose (kdst = Vp); with WT null, W is read as
// stored and G_c is the memory-lean backward's tile (lean: stage-tiled for bf16, K-blocked for
// fp32) or row-major [cc][ldg]. Split over the vocabulary into n_split fp32 partials when
// n_split > 1 (part: [n_split][cc][d]), then reduced in a fixed order.
hipError_t launch_dh(const Shape& sh, const void* Gc, int64_t ldg, const void* W, const void* WT,
                     int64_t c0, int64_t cc, int n_split, float* part, void* dH, hipStream_t s,
                     bool lean = false);

// dW (+)= G_c^T H[c0:c0+cc] from G_c and H, both M/N contiguous: G_c row-major [cc][ldg], or
// the memory-lean backward's tile (lean; ldg unused): stage-tiled for bf16 (wide tiles, LDS
// transpose reads), K-blocked [Vp/256][cc][256] for fp32.
hipError_t launch_dw(const Shape& sh, const void* Gc, int64_t ldg, const void* H, int64_t c0,
                     int64_t cc, bool accumulate, float* dW, hipStream_t s, bool lean = false);
// dW (+)= G_c^T H_c over K columns [0, cc) from stage-tiled G_c^T (launch_bwd_grad, ldgt K
// columns) and H_c^T (launch_transpose, kdst = ldht).
hipError_t launch_dw_t(const Shape& sh, const void* GT, int64_t ldgt, const void* HT, int64_t ldht,
                       int64_t cc, bool accumulate, float* dW, hipStream_t s);

// Dense path pieces.
hipError_t launch_dense_logits(const Shape& sh, const void* H, const void* W, float* Z, int64_t ldz,
                               hipStream_t s);
hipError_t launch_dense_rows(const Shape& sh, float* Z, float* P, int64_t ldz, const int32_t* idx,
                             const void* tlog, const float* grad_loss, float* lse, float* row_kl,
                             double* row_sum, void* G, int64_t ldg, hipStream_t s);
hipError_t launch_sum_rows(const Shape& sh, const double* row_sum, double* blk_sum, int* n_blk,
                           hipStream_t s);

int64_t round_up(int64_t x, int64_t m);
int dh_splits(int64_t cc, int64_t d, int64_t V, bool wide);  // wide: 320-column dH tiles
int fwd_vsplits(int64_t N, int64_t V);

}  // namespace kdkl
