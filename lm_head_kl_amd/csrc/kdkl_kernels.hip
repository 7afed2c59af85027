// HIP kernels of libkdkl for gfx950 (MI355X): the fused chunked top-K KL loss over the LM head.
//
// What is computed follows the pages' description of the fused chunked KL loss:
// "Making knowledge distillation cheap enough to run in production" (aiexpert.news),
// paragraph on the second fix. The hidden states are projected to logits one piece at a
// time; each piece is folded into a running loss accumulator and then discarded; the
// backward pass recomputes each piece. The teacher side is the top-K cache from the
// paragraph on the first fix.
//
// Every GEMM-shaped kernel runs on the MFMA tile engine of engine.h. A workgroup owns a fp32
// tile of C = A B^T with its accumulators in registers:
//   - forward and gradient kernels: 256 x 256, eight 64-wide waves in a 2 x 4 grid, each wave
//     128 x 64 as 8 x 4 blocks of v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x4_f32 for fp32);
//   - dH and dW: 256 x 320 (the hidden size on the 320 side), eight waves of 128 x 80, also
//     in the bf16 memory-lean backward;
//   - the dense comparison path and the fp32 memory-lean backward: 256 x 256 on four waves of
//     32x32x16 blocks.
// Operands reach LDS straight from memory (buffer_load ... lds) in 16-byte chunks, XOR-swizzled
// by row so that fragment reads are free of bank conflicts, four stages of half a K step deep.
// Every operand of the fast path is stage-tiled (engine.h, kTiled): each 64-byte K step of a
// tile's rows is one contiguous block, so its loads fetch whole 128-byte lines. The copies are
// made here: for the forward, W and each launch's rows of H (k_tile_rows); for the backward,
// W^T once per call and H_c^T per chunk (k_transpose), whose loads also write the gradient
// kernel's stage-tiled W and H_c; and G_c and G_c^T, written by the gradient kernels. The bf16
// memory-lean backward makes no copy: dH and dW read W, H and the stage-tiled G_c through LDS
// transpose reads (engine.h, kTrans / kTransT). The dense path and the fp32 memory-lean
// backward read row-major or M/N-contiguous operands through registers (8 x 8 blocks transposed
// on the way to LDS).
//
// Epilogues:
//   forward   logit tiles are computed transposed (vocabulary x tokens), so each lane keeps the
//             running (max, sum) of its token columns in the log2 domain without shuffles; the
//             gather of z at the cached ids goes through an LDS-staged half tile;
//   backward  G = g*T/n_norm*(softmax(z/T) - P_t), P_t subtracted in the LDS-staged tile, then
//             stored twice in the activation dtype, stage-tiled: G_c for dH and G_c^T for dW;
//   dH        fp32 split-K partials, reduced in a fixed order, or a direct store;
//   dW        fp32 read-modify-write through LDS.
// Hand-offs of staged LDS data inside an epilogue use an LDS-only barrier: a full workgroup
// barrier would also wait for the global stores already issued.
//
// MFMA lane layouts (checked on gfx950 hardware):
//   32x32x16 bf16: lane l supplies A[m = l%32][k = 8*(l/32) + 0..7], B likewise with n.
//   32x32x2 f32:   lane l supplies A[m = l%32][k = l/32].
//   Accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
//   16x16x32 bf16: lane l supplies A[m = l%16][k = 8*(l/16) + 0..7]; accumulator element v of
//                  lane l: row 4*(l/16) + v, column l%16.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "engine.h"
#include "kdkl_internal.h"

namespace kdkl {

#define KD_LAUNCH(kind, stream, ...)         \
    do {                                     \
        timing_begin(kind, stream);          \
        hipLaunchKernelGGL(__VA_ARGS__);     \
        timing_end(kind, stream);            \
    } while (0)

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float load_t(const void* p, Dt dt, int64_t i) {
    return dt == Dt::BF16 ? bf2f(((const bf16_t*)p)[i]) : ((const float*)p)[i];
}

// Merge (m2, s2) into (m, s): sums of 2^(y - m) over disjoint sets.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = s * exp2_fast(m - M) + s2 * exp2_fast(m2 - M);
    m = M;
}

template <int HALF, int MASK, int NPOS>
__device__ __forceinline__ void rs_step(float (&pm)[NPOS], float (&ps)[NPOS], int lane) {
    const bool up = (lane & MASK) != 0;
#pragma unroll
    for (int q = 0; q < HALF; ++q) {
        float km = up ? pm[q + HALF] : pm[q];
        float ks = up ? ps[q + HALF] : ps[q];
        const float sm = up ? pm[q] : pm[q + HALF];
        const float ss = up ? ps[q] : ps[q + HALF];
        const float rm = __shfl_xor(sm, MASK);
        const float rsum = __shfl_xor(ss, MASK);
        ms_merge(km, ks, rm, rsum);
        pm[q] = km;
        ps[q] = ks;
    }
}

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Row of accumulator element e of lane half h inside its 32 x 32 MFMA block.
__device__ __forceinline__ int blk_row(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

// Element offset of (row, k) in a stage-tiled operand (engine.h, kTiled) with row blocks of RB
// rows and S stages of SW = 64 bytes per row block.
template <typename T, int RB>
__device__ __forceinline__ int64_t tiled_at(int64_t row, int64_t k, int64_t S) {
    constexpr int SW = 64 / (int)sizeof(T);
    return ((row / RB) * S + k / SW) * (int64_t)(RB * SW) + (row % RB) * SW + k % SW;
}

// Staging of half a transposed tile in LDS: 128 rows (vocabulary entries) x 256 columns
// (tokens) of fp32. Stage row sr holds tile row (sr/64)*128 + pass*64 + sr%64. Column t of row
// r sits at t ^ st_swz(r); the XOR touches bits 2..5 only, so runs of 4 columns stay
// contiguous and 16-byte aligned. With 64 four-byte banks it is conflict free for the
// accumulator writes of 16 x 16 blocks (rows r, r+4, r+8, r+12 by 16 tokens: bits 4..5 of the
// XOR differ) and for column reads of 16 rows 8 apart by 4 tokens (bits 2..5 differ).
constexpr int SST = kTileN;
__device__ __forceinline__ int st_swz(int r) { return (((r >> 3) ^ (((r >> 2) & 3) << 2)) & 15) << 2; }
__device__ __forceinline__ int st_idx(int r, int t) { return r * SST + (t ^ st_swz(r)); }
// Stage row of tile row c in the pass that holds it (pass (c >> 6) & 1).
__device__ __forceinline__ int st_row(int c) { return (c >> 7) * 64 + (c & 63); }

// ------------------------------------------------------------------------------------------
// Plan: bucket cached ids by (row block of 256, vocab tile of 256).

// One workgroup of kPlanThreads per row block: the grid is only N / 256 workgroups, so each
// one is wide, and the bucket offsets come from a shuffle scan rather than a serial one.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ idx, int64_t row0,
                                                       int64_t row1, int K, int64_t V, int n_vt,
                                                       int32_t* __restrict__ off, uint32_t* __restrict__ ent) {
    constexpr int PT = kPlanThreads, PW = PT / 64;
    __shared__ int cnt[kMaxVTiles];
    __shared__ int wsum[PW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rb = blockIdx.x;
    const int64_t r0 = row0 + (int64_t)rb * kTileM;
    const int rows = (int)min<int64_t>(kTileM, row1 - r0);
    const int64_t base = (int64_t)rb * kTileM * K;
    for (int t = tid; t < n_vt; t += PT) cnt[t] = 0;
    __syncthreads();
    const int n_e = rows * K;
    // Entries go in batches of PB per thread, all loaded before any is used, so the loads'
    // latency is paid once per batch rather than once per entry.
    constexpr int PB = 8;
    for (int i0 = 0; i0 < n_e; i0 += PT * PB) {
        int v[PB];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int i = i0 + u * PT + tid;
            v[u] = i < n_e ? idx[r0 * K + i] : -1;
        }
#pragma unroll
        for (int u = 0; u < PB; ++u)
            if (v[u] >= 0 && v[u] < V) atomicAdd(&cnt[v[u] >> 8], 1);
    }
    __syncthreads();
    // Exclusive scan of cnt[0..n_vt): each thread owns a contiguous segment; the segment sums
    // are scanned within each wave by shuffles, then across the PW wave totals.
    const int seg = (n_vt + PT - 1) / PT;
    const int s0 = min(n_vt, tid * seg), s1 = min(n_vt, s0 + seg);
    int sum = 0;
    for (int t = s0; t < s1; ++t) sum += cnt[t];
    int incl = sum;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const int y = __shfl_up(incl, m);
        if (lane >= m) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (tid < 64) {
        const int x = lane < PW ? wsum[lane] : 0;
        int wi = x;
#pragma unroll
        for (int m = 1; m < PW; m <<= 1) {
            const int y = __shfl_up(wi, m);
            if (lane >= m) wi += y;
        }
        if (lane < PW) wsum[lane] = wi - x;
    }
    __syncthreads();
    int run = wsum[w] + incl - sum;
    int32_t* o = off + (int64_t)rb * (n_vt + 1);
    for (int t = s0; t < s1; ++t) {
        const int x = cnt[t];
        cnt[t] = run;  // becomes the fill cursor
        o[t] = (int32_t)(base + run);
        run += x;
    }
    if (tid == PT - 1) o[n_vt] = (int32_t)(base + run);  // the last segment ends at the total
    __syncthreads();
    for (int i0 = 0; i0 < n_e; i0 += PT * PB) {
        int v[PB];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int i = i0 + u * PT + tid;
            v[u] = i < n_e ? idx[r0 * K + i] : -1;
        }
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            if (v[u] >= 0 && v[u] < V) {
                const int i = i0 + u * PT + tid;
                const int pos = atomicAdd(&cnt[v[u] >> 8], 1);
                const int r = i / K, k = i - r * K;
                ent[base + pos] = (uint32_t)r | ((uint32_t)(v[u] & 255) << 8) | ((uint32_t)k << 16);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Teacher probabilities: p_t = softmax(t/T) over the K cached entries (one wave per row).

__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmax(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

__global__ __launch_bounds__(256) void k_teacher_prob(const void* __restrict__ tlog, Dt tdt, int64_t row0,
                                                      int64_t row1, int K, float T, float* __restrict__ pt) {
    const int lane = threadIdx.x & 63;
    const int64_t n = row0 + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= row1) return;
    double mx = -INFINITY;
    for (int k = lane; k < K; k += 64) mx = fmax(mx, (double)load_t(tlog, tdt, n * K + k) / T);
    mx = wave_max_d(mx);
    double s = 0.0;
    for (int k = lane; k < K; k += 64) s += exp((double)load_t(tlog, tdt, n * K + k) / T - mx);
    const double lz = mx + log(wave_sum_d(s));
    float* o = pt + (n - row0) * K;
    for (int k = lane; k < K; k += 64) o[k] = (float)exp((double)load_t(tlog, tdt, n * K + k) / T - lz);
}

// ------------------------------------------------------------------------------------------
// Id validation: range and distinctness within each row (one wave per row).

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_validate(const int32_t* __restrict__ idx, int64_t N, int K, int64_t V,
                                                  uint32_t* status) {
    __shared__ int ids[4][kMaxK];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t n = (int64_t)blockIdx.x * 4 + w;
    const bool live = n < N;
    uint32_t bad = 0;
    for (int k = lane; k < K; k += 64) {
        const int v = live ? idx[n * K + k] : 0;
        ids[w][k] = v;
        if (live && (v < 0 || v >= V)) bad |= 1u;
    }
    __syncthreads();
    if (live) {
        for (int k = lane; k < K; k += 64) {
            const int v = ids[w][k];
            for (int j = 0; j < K; ++j)
                if (j != k && ids[w][j] == v) bad |= 2u;
        }
    }
    if (bad) atomicOr(status, bad);
}

// ------------------------------------------------------------------------------------------
// Fused forward.

struct FwdArgs {
    const void* H;  // row-major [N][d], or stage-tiled (ldh stages per row block)
    const void* W;  // row-major [V][d], or stage-tiled (ldw stages per row block)
    int64_t ldh, ldw;
    int64_t N, d, V, K;
    float c;  // log2(e)/T
    const int32_t* off;
    const uint32_t* ent;
    int n_vt;
    int Q;          // vocab lanes: unit (rb, q) takes vocab tiles q, q + Q, q + 2Q, ...
    int64_t n_unit; // row blocks * Q
    float2* part;   // [2Q][N]: per (lane, wave row) partial (max, sum) of each row
    float* zk;
    float* zt;      // if not null, the logits are also stored transposed: z^T [Vp][ldzt]
    int64_t ldzt;
};

// Persistent forward. Units (row block, vocab lane) are ordered row-block major. XCD x
// takes the contiguous band [x*band, (x+1)*band), so its 32 workgroups work on a few row
// blocks times Q vocab lanes at once. Those share both the H rows and the W tiles in the
// XCD's L2.
//
// The tile is computed transposed, z^T = W_tile H_block^T: accumulator rows are vocabulary
// entries and columns are tokens. Each lane then holds 64 vocabulary entries of each of its
// 4 token columns, so the per-token (max, sum) over the vocabulary is folded inside the lane,
// and lanes only meet once per unit.
template <typename T, bool ZT, int NW, int LAY>
__global__ __launch_bounds__(64 * NW, 1) void k_fwd(FwdArgs a) {
    static_assert(NW == 8, "the forward runs on eight waves with 16 x 16 blocks");
    constexpr int NT = 64 * NW;
    __shared__ u32x4 L[LDS_CHUNKS];
    const WaveIdN<NW> id;
    const int64_t P = gridDim.x;
    const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd = P / 8;
    const int64_t band = (a.n_unit + 7) / 8;
    const int64_t u_end = min(a.n_unit, (xcd + 1) * band);
    float* stage = (float*)L;

    for (int64_t u = xcd * band + slot; u < u_end; u += per_xcd) {
        const int rb = (int)(u / a.Q), q = (int)(u % a.Q);
        const int64_t m0 = (int64_t)rb * kTileM;  // first token of the row block
        const int32_t* off = a.off + (int64_t)rb * (a.n_vt + 1);
        // Running (max, sum) in units of y = z*log2(e)/T for this lane's 4 token columns
        // wn*64 + 16j + lane%16, over the vocabulary rows the lane holds.
        float run_m[4], run_s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            run_m[j] = -INFINITY;
            run_s[j] = 0.f;
        }

        for (int vt = q; vt < a.n_vt; vt += a.Q) {
            const int64_t n0 = (int64_t)vt * kTileN;
            // The tile's first NT cached-id entries go to registers (one per thread) before the
            // mainloop, so their load latency hides behind it.
            const int e0 = off[vt], e1 = off[vt + 1];
            const uint32_t my_en = e0 + id.tid < e1 ? a.ent[e0 + id.tid] : 0xffffffffu;
            f32x4 acc[8][4];
            gemm_tile_kk16<T, LAY, LAY>(acc, L, id, (const T*)a.W, a.ldw, n0, a.V, a.d, (const T*)a.H, a.ldh, m0,
                                        a.N, a.d, 0, a.d);
            const WaveIdN<NW> ie = id.fresh();
            const int g4 = 4 * (ie.lane >> 4), c16 = ie.lane & 15;

            // Gather z at the cached ids of this (row block, vocab tile): two passes of 128
            // vocabulary rows staged in LDS. The paths that keep the logits also store the
            // staged rows as z^T, a wave writing 1 KB of one row per step.
            if (ZT || e1 > e0) {
#pragma unroll
                for (int pq = 0; pq < 2; ++pq) {
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int sr = ie.wm * 64 + 16 * i4 + g4 + v;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                stage[st_idx(sr, ie.wn * 64 + 16 * j + c16)] = acc[4 * pq + i4][j][v];
                        }
                    lds_barrier();
                    if (my_en != 0xffffffffu && ((my_en >> 14) & 1) == (uint32_t)pq) {
                        const int r = my_en & 255, c = (my_en >> 8) & 255, k = (int)(my_en >> 16);
                        a.zk[(m0 + r) * a.K + k] = stage[st_idx(st_row(c), r)];
                    }
                    for (int i = e0 + NT + ie.tid; i < e1; i += NT) {
                        const uint32_t en = a.ent[i];
                        const int c = (en >> 8) & 255;
                        if (((c >> 6) & 1) != pq) continue;
                        const int r = en & 255, k = (int)(en >> 16);
                        a.zk[(m0 + r) * a.K + k] = stage[st_idx(st_row(c), r)];
                    }
                    if constexpr (ZT) {
#pragma unroll 8
                        for (int k = 0; k < 8192 / NT; ++k) {
                            const int it = ie.tid + NT * k;
                            const int sr = it >> 6, tok = (it & 63) * 4;
                            const int64_t v = n0 + (sr >> 6) * 128 + pq * 64 + (sr & 63);
                            if (v < a.V && m0 + tok < a.N)
                                *(f32x4*)(a.zt + v * a.ldzt + m0 + tok) = *(const f32x4*)(stage + st_idx(sr, tok));
                        }
                    }
                    lds_barrier();
                }
            }

            // Tile (max, sum) per token column, folded over the lane's 32 vocabulary rows, then
            // merged into the running pair. Rows past V (last tile only) count as -inf.
            const bool vfull = n0 + kTileN <= a.V;
            const int rows_left = (int)min<int64_t>(kTileN, a.V - n0) - ie.wm * 128 - g4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const bool ok = vfull || 16 * i + v < rows_left;
                        mx = fmaxf(mx, ok ? acc[i][j][v] : -INFINITY);
                    }
                const float mt = mx * a.c;
                float s = 0.f;
                if (mx != -INFINITY) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const bool ok = vfull || 16 * i + v < rows_left;
                            s += ok ? exp2_fast(fmaf(acc[i][j][v], a.c, -mt)) : 0.f;
                        }
                }
                ms_merge(run_m[j], run_s[j], mt, s);
            }
        }

        // Lanes l, l^16, l^32, l^48 hold the same token columns over different vocabulary rows.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float m2 = __shfl_xor(run_m[j], 16), s2 = __shfl_xor(run_s[j], 16);
            ms_merge(run_m[j], run_s[j], m2, s2);
            m2 = __shfl_xor(run_m[j], 32);
            s2 = __shfl_xor(run_s[j], 32);
            ms_merge(run_m[j], run_s[j], m2, s2);
        }
        if (id.lane < 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t g = m0 + id.wn * 64 + 16 * j + id.lane;
                if (g < a.N) a.part[(int64_t)(q * 2 + id.wm) * a.N + g] = make_float2(run_m[j], run_s[j]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Combine: lse_n from the partials, KL_n from the cached teacher and zk, block sums in fp64.

constexpr int kCombRows = 4;  // rows per workgroup (one per wave: each row is a chain of dependent reductions)

__global__ __launch_bounds__(256) void k_combine(const float2* __restrict__ part, int n_part, int64_t N, int K,
                                                 float T, const float* __restrict__ zk,
                                                 const void* __restrict__ tlog, Dt tdt, float* __restrict__ lse,
                                                 float* __restrict__ row_kl, double* __restrict__ blk_sum) {
    __shared__ double wsum[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double mine = 0.0;
    for (int rr = 0; rr < kCombRows / 4; ++rr) {
        const int64_t n = (int64_t)blockIdx.x * kCombRows + w * (kCombRows / 4) + rr;
        if (n >= N) break;
        const void* tl = tlog;
        auto tval = [&](int k) { return (double)load_t(tl, tdt, n * K + k) / T; };
        // The row's first 128 cached entries are loaded once, up front, beside the partials;
        // entries past 128 (K > 128) are read in each pass. Every sum runs in the same order
        // over k either way.
        double tv[2];
        float zv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int k = lane + 64 * j;
            tv[j] = k < K ? tval(k) : 0.0;
            zv[j] = k < K ? zk[n * K + k] : 0.f;
        }
        float m = -INFINITY, s = 0.f;
        for (int sl = lane; sl < n_part; sl += 64) {
            const float2 v = part[(int64_t)sl * N + n];
            if (v.y > 0.f) ms_merge(m, s, v.x, v.y);
        }
#pragma unroll
        for (int mk = 32; mk >= 1; mk >>= 1) {
            const float m2 = __shfl_xor(m, mk), s2 = __shfl_xor(s, mk);
            ms_merge(m, s, m2, s2);
        }
        const double lse_d = ((double)m + log2((double)s)) * kLn2;
        double mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (lane + 64 * j < K) mx = fmax(mx, tv[j]);
        for (int k = lane + 128; k < K; k += 64) mx = fmax(mx, tval(k));
        mx = wave_max_d(mx);
        double se = 0.0;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (lane + 64 * j < K) se += exp(tv[j] - mx);
        for (int k = lane + 128; k < K; k += 64) se += exp(tval(k) - mx);
        const double lz = mx + log(wave_sum_d(se));
        // An entry whose teacher logit is -inf has p_t = 0 and adds nothing (0 log 0 = 0).
        double term = 0.0;
        auto add_term = [&](double t, float z) {
            const double lp = t - lz;
            const double pk = exp(lp);
            if (pk > 0.0) term += pk * (lp - (double)z / T + lse_d);
        };
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (lane + 64 * j < K) add_term(tv[j], zv[j]);
        for (int k = lane + 128; k < K; k += 64) add_term(tval(k), zk[n * K + k]);
        const double kl = wave_sum_d(term);
        if (lane == 0) {
            lse[n] = (float)lse_d;
            if (row_kl) row_kl[n] = (float)kl;
        }
        mine += kl;
    }
    if (lane == 0) wsum[w] = mine;
    __syncthreads();
    if (threadIdx.x == 0) blk_sum[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

__global__ __launch_bounds__(256) void k_loss_final(const double* __restrict__ blk_sum, int n_blk, double scale,
                                                    float* __restrict__ loss) {
    __shared__ double red[NTHR];
    double s = 0.0;
    for (int i = threadIdx.x; i < n_blk; i += NTHR) s += blk_sum[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = NTHR / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = (float)(scale * red[0]);
}

// Per-row fp64 values summed into block partials in a fixed order (dense path).
__global__ __launch_bounds__(256) void k_sum_rows(const double* __restrict__ v, int64_t N, double* __restrict__ blk) {
    __shared__ double red[NTHR];
    const int64_t i0 = (int64_t)blockIdx.x * 1024;
    double s = 0.0;
    for (int t = 0; t < 4; ++t) {
        const int64_t i = i0 + t * NTHR + threadIdx.x;
        if (i < N) s += v[i];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = NTHR / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) blk[blockIdx.x] = red[0];
}

// ------------------------------------------------------------------------------------------
// Backward, per chunk: recompute the logit tile and form G = gs*(2^(y - lse2) - P_t).
//
// Like the forward, the tile is computed transposed (rows: vocabulary entries, columns:
// tokens), so each lane needs the lse of only its 4 token columns, kept in registers. The
// tile leaves through LDS in two passes of 128 vocabulary rows, which lets both copies be
// written in whole 128-byte lines: G (a token's entries of the pass, 64 bytes in each of four
// stage blocks, the neighbouring token completing each line) and G^T (a vocabulary entry's 256
// consecutive tokens).

struct GradArgs {
    const void* H;  // row-major [N][d], or stage-tiled (ldh stages per row block)
    const void* W;  // row-major [V][d], or stage-tiled (ldw stages per row block)
    int64_t ldh, ldw;
    int64_t d, V, K;
    float c;      // log2(e)/T
    float gsc;    // T/n_norm
    const float* grad;  // device scalar or nullptr
    const float* lse;
    const float* pt;    // [cc][K], rows relative to c0
    int64_t c0, cc;
    const int32_t* off;
    const uint32_t* ent;
    int n_vt, n_rbc;
    // G_c, rows = the chunk's tokens, K = vocabulary: stage-tiled (row blocks of 256, Vp/SW
    // stages), or K-blocked [Vp/256][cc][256] (entry (t, v) at ((v/256)*cc + t)*256 + v%256)
    void* G;
    // G_c^T, rows = vocabulary, K = tokens of the dW group: stage-tiled (row blocks of 256, ldgt/SW
    // stages), the chunk's tokens at K columns gt_col0 .. gt_col0 + cc, zero up to gt_col0 + ccp;
    // nullptr to skip
    void* GT;
    int64_t ldgt, ccp, gt_col0;
    const float* zt;  // stored logits z^T [Vp][ldzt] (k_grad_z), chunk columns from zt_col0
    int64_t ldzt, zt_col0;
};

// Non-temporal: G and G^T (1.65 GB per chunk) would otherwise evict the W and H_c lines the
// next tiles' operand loads hit in L2 (about 1% faster gradient kernel).
template <typename T>
__device__ __forceinline__ void store8(T* dst, const float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        u32x4 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = pack_bf16x2(x[2 * u], x[2 * u + 1]);
        __builtin_nontemporal_store(o, (u32x4*)dst);
    } else {
        __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4*)dst);
        __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, (f32x4*)(dst + 4));
    }
}

// Second half of a gradient pass, once the pass's 128 vocabulary rows of gs*softmax are staged:
// subtract gs*p_t at the cached ids that fall in the pass, then write the rows of G (stage-tiled,
// or K-blocked for the fp32 memory-lean backward) and of G^T. Ends with a barrier, so the stage may be
// refilled.
// The plan fills each bucket in atomic order, so whether an entry is among the first NT (held
// in registers) or comes from the loop changes between calls; both paths subtract with one
// explicit fused multiply-add, so G does not depend on that order.
template <typename T, int NW, int GL>
__device__ __forceinline__ void grad_pass_out(const GradArgs& a, float* stage, int pq, const WaveIdN<NW>& ie, int vt,
                                              int64_t r0, int64_t n0, int e0, int e1, uint32_t my_en, float my_pt,
                                              float gs) {
    constexpr int SW = 64 / (int)sizeof(T);
    constexpr int NT = 64 * NW, IT = 4096 / NT;  // items per thread of each output layout
    if (my_en != 0xffffffffu && ((my_en >> 14) & 1) == (uint32_t)pq) {
        const int r = my_en & 255, c = (my_en >> 8) & 255;
        float& x = stage[st_idx(st_row(c), r)];
        x = fmaf(-gs, my_pt, x);
    }
    for (int i = e0 + NT + ie.tid; i < e1; i += NT) {
        const uint32_t en = a.ent[i];
        const int c = (en >> 8) & 255;
        if (((c >> 6) & 1) != pq) continue;
        const int r = en & 255, k = (int)(en >> 16);
        float& x = stage[st_idx(st_row(c), r)];
        x = fmaf(-gs, a.pt[(r0 + r) * a.K + k], x);
    }
    lds_barrier();
    if constexpr (GL == kTiled) {
        // Stage-tiled G rows: token tl, group g of 8 vocabulary entries (stage rows 8g .. 8g+7,
        // read one by one); 16 lanes write a token's 128 entries of the pass, 64 bytes in each of
        // four stage blocks, and the next 16 lanes the next token's, the other half of each
        // 128-byte line.
#pragma unroll 4
        for (int q = 0; q < 4096 / NT; ++q) {
            const int it = ie.tid + NT * q;
            const int g = it & 15, tl = it >> 4;
            const int64_t tr = r0 + tl;
            if (tr < a.cc) {
                float x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = stage[st_idx(8 * g + u, tl)];
                const int vb = (g >> 3) * 128 + pq * 64 + (g & 7) * 8;
                store8<T>((T*)a.G + tiled_at<T, kTileM>(tr, n0 + vb, (int64_t)a.n_vt * (kTileN / SW)), x);
            }
        }
    } else {
    // G rows: group g of 8 vocabulary entries (stage rows 8g .. 8g+7) by a group of 4 tokens.
    // A lane reads the 8 x 4 block with 16-byte LDS reads (4 tokens of one stage row each) and
    // writes the 4 tokens' 8-entry segments; 16 consecutive lanes cover one token's 128
    // entries of the pass: two whole 128-byte lines.
#pragma unroll 2
    for (int ib = 0; ib < 1024 / NT; ++ib) {
        const int it = ie.tid + NT * ib;
        const int g = it & 15, tq = it >> 4;
        f32x4 blk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) blk[u] = *(const f32x4*)(stage + st_idx(8 * g + u, 4 * tq));
        const int vb = (g >> 3) * 128 + pq * 64 + (g & 7) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t tr = r0 + 4 * tq + j;
            if (tr < a.cc) {
                const float x[8] = {blk[0][j], blk[1][j], blk[2][j], blk[3][j],
                                    blk[4][j], blk[5][j], blk[6][j], blk[7][j]};
                store8<T>((T*)a.G + ((int64_t)vt * a.cc + tr) * kTileN + vb, x);
            }
        }
    }
    }
    // G^T rows: vocabulary entry of stage row sr, group cb of 8 tokens; 32 lanes write a row's
    // 256 tokens.
    if (a.GT) {
#pragma unroll 4
        for (int it8 = 0; it8 < IT; ++it8) {
            const int it = ie.tid + NT * it8;
            const int sr = it >> 5, cb = it & 31;
            const int64_t tr = r0 + cb * 8;
            if (tr < a.ccp) {
                const float* row = stage + sr * SST;
                const f32x4 v0 = *(const f32x4*)(row + ((cb * 8) ^ st_swz(sr)));
                const f32x4 v1 = *(const f32x4*)(row + ((cb * 8 + 4) ^ st_swz(sr)));
                const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                const int vr = (sr >> 6) * 128 + pq * 64 + (sr & 63);
                store8<T>((T*)a.GT + tiled_at<T, kTileM>(n0 + vr, a.gt_col0 + tr, a.ldgt / SW), x);
            }
        }
    }
    lds_barrier();
}

template <typename T, int NW, int LAY, int GL>
__global__ __launch_bounds__(64 * NW, 1) void k_bwd_grad(GradArgs a) {
    static_assert(NW == 8, "the gradient kernel runs on eight waves with 16 x 16 blocks");
    constexpr int NT = 64 * NW;
    __shared__ u32x4 L[LDS_CHUNKS];
    const WaveIdN<NW> id;
    // Persistent when launched with fewer workgroups than tiles. Logical tiles are vocab-tile
    // major; XCD x owns the contiguous band [x*band, (x+1)*band) and walks it with stride
    // per_xcd, so the tiles in flight on one XCD are a few W tiles times every row block of
    // the chunk, which share operand lines in the XCD's L2.
    const int64_t n_tiles = (int64_t)a.n_vt * a.n_rbc;
    const int64_t band = (n_tiles + 7) / 8, per_xcd = gridDim.x / 8;
    const int64_t t_beg = (blockIdx.x % 8) * band, t_end = min(n_tiles, t_beg + band);
    float* stage = (float*)L;
    // The chunk's first row of H: row c0 of row-major H; a stage-tiled H holds the chunk alone.
    const T* Hc = LAY == kTiled ? (const T*)a.H : (const T*)a.H + a.c0 * a.ldh;
    for (int64_t t = t_beg + blockIdx.x / 8; t < t_end; t += per_xcd) {
        const int vt = (int)(t / a.n_rbc), rb = (int)(t % a.n_rbc);
        const int64_t r0 = (int64_t)rb * kTileM;  // token offset within the chunk
        const int64_t n0 = (int64_t)vt * kTileN;
        const float gs = (a.grad ? a.grad[0] : 1.f) * a.gsc;
        // Everything below up to the mainloop is needed only by the epilogue: the loads are
        // issued without branches so that their latency hides behind the mainloop's first DMA
        // stages instead of being waited for one by one.
        // lse of the lane's 4 token columns wn*64 + 16j + lane%16 (a clamped index past the chunk)
        float lse_raw[4];
        bool tok_ok[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t tr = r0 + id.wn * 64 + 16 * j + (id.lane & 15);
            tok_ok[j] = tr < a.cc;
            lse_raw[j] = a.lse[a.c0 + (tok_ok[j] ? tr : 0)];
        }
        // This tile's cached-id entries: the first NT are loaded into registers (one per
        // thread) before the mainloop; more only occur on Zipf-hot tiles. Their p_t is
        // loaded after the mainloop, ahead of its first use.
        const int32_t* off = a.off + (int64_t)rb * (a.n_vt + 1);
        const int e0 = off[vt], e1 = off[vt + 1];
        const bool has_en = e0 + id.tid < e1;
        const uint32_t my_en = a.ent[has_en ? e0 + id.tid : 0] | (has_en ? 0u : 0xffffffffu);
        f32x4 acc[8][4];
        gemm_tile_kk16<T, LAY, LAY>(acc, L, id, (const T*)a.W, a.ldw, n0, a.V, a.d, Hc, a.ldh, r0, a.cc, a.d, 0,
                                    a.d);
        const float my_pt = my_en != 0xffffffffu ? a.pt[(r0 + (my_en & 255)) * a.K + (my_en >> 16)] : 0.f;
        float l2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) l2[j] = tok_ok[j] ? lse_raw[j] * kLog2e : 0.f;
        const WaveIdN<NW> ie = id.fresh();
        const int g4 = 4 * (ie.lane >> 4), c16 = ie.lane & 15;

#pragma unroll
        for (int pq = 0; pq < 2; ++pq) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int i = 4 * pq + i4;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool vok = n0 + ie.wm * 128 + 16 * i + g4 + v < a.V;
                    const int sr = ie.wm * 64 + 16 * i4 + g4 + v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x = (vok && tok_ok[j]) ? gs * exp2_fast(fmaf(acc[i][j][v], a.c, -l2[j])) : 0.f;
                        stage[st_idx(sr, ie.wn * 64 + 16 * j + c16)] = x;
                    }
                }
            }
            lds_barrier();
            grad_pass_out<T, NW, GL>(a, stage, pq, ie, vt, r0, n0, e0, e1, my_en, my_pt, gs);
        }
    }
}

// Gradient tile from stored logits z^T (forward-chunked and single-pass paths): the same G and
// G^T as k_bwd_grad, with the tile read from memory instead of recomputed. HBM-bound: it reads
// 4 bytes and writes 2 x 2 bytes per entry. The tile goes through LDS in four passes of 64
// vocabulary rows (64 KB), so two workgroups share a CU and the loads of one overlap the
// stores of the other; each pass's z^T rows are requested before the previous pass is staged.
// G is formed with the same operations as in k_bwd_grad (the exp2 of the tempered logit minus
// lse, times gs, then gs*p_t subtracted with one fused multiply-add), so both kernels give the
// same bits.
constexpr int kGzRows = 64;  // vocabulary rows per pass

template <typename T>
__global__ __launch_bounds__(256, 2) void k_grad_z(GradArgs a) {
    constexpr int IT = kGzRows * kTileM / 4 / NTHR;  // 16-byte items per thread per pass (16)
    constexpr int SW = 64 / (int)sizeof(T);
    __shared__ u32x4 L[kGzRows * SST / 4 + kTileM / 4];
    float* stage = (float*)L;
    float* lse2 = (float*)(L + kGzRows * SST / 4);
    const WaveId id;
    const int64_t n_tiles = (int64_t)a.n_vt * a.n_rbc;
    const int64_t t = xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles) return;
    const int vt = (int)(t / a.n_rbc), rb = (int)(t % a.n_rbc);
    const int64_t r0 = (int64_t)rb * kTileM;
    const int64_t n0 = (int64_t)vt * kTileN;
    {
        const int64_t r = r0 + id.tid;
        lse2[id.tid] = r < a.cc ? a.lse[a.c0 + r] * kLog2e : 0.f;
    }
    const float gs = (a.grad ? a.grad[0] : 1.f) * a.gsc;
    const int32_t* off = a.off + (int64_t)rb * (a.n_vt + 1);
    const int e0 = off[vt], e1 = off[vt + 1];
    uint32_t my_en = 0xffffffffu;
    float my_pt = 0.f;
    if (e0 + id.tid < e1) {
        my_en = a.ent[e0 + id.tid];
        my_pt = a.pt[(r0 + (my_en & 255)) * a.K + (my_en >> 16)];
    }
    // Vector loads when every chunk column offset is 16-byte aligned (uniform).
    const bool vec = ((a.ldzt | (a.zt_col0 + r0)) & 3) == 0;
    // Pass pq holds tile rows pq*64 .. pq*64+63; item k of a thread is stage row it/64, tokens
    // 4*(it%64) .. +3, so a wave reads 1 KB of one z^T row per item.
    auto load = [&](int pq, f32x4 (&z)[IT]) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = id.tid + NTHR * k;
            const int sr = it >> 6, tok = (it & 63) * 4;
            const int64_t v = n0 + pq * kGzRows + sr;
            z[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (v < a.V && r0 + tok < a.cc) {
                const float* zr = a.zt + v * a.ldzt + a.zt_col0 + r0 + tok;
                if (vec) {
                    z[k] = *(const f32x4*)zr;
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (r0 + tok + u < a.cc) z[k][u] = zr[u];
                }
            }
        }
    };
    auto pass = [&](int pq, const f32x4 (&z)[IT]) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = id.tid + NTHR * k;
            const int sr = it >> 6, tok = (it & 63) * 4;
            const int64_t v = n0 + pq * kGzRows + sr;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            if (v < a.V) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (r0 + tok + u < a.cc) g[u] = gs * exp2_fast(fmaf(z[k][u], a.c, -lse2[tok + u]));
            }
            *(f32x4*)(stage + st_idx(sr, tok)) = g;
        }
        lds_barrier();
        // gs*p_t at the cached ids whose vocabulary row is in this pass (bits 6-7 of the column)
        if (my_en != 0xffffffffu && ((my_en >> 14) & 3) == (uint32_t)pq) {
            const int r = my_en & 255, c = (my_en >> 8) & 255;
            float& x = stage[st_idx(c & 63, r)];
            x = fmaf(-gs, my_pt, x);
        }
        for (int i = e0 + NTHR + id.tid; i < e1; i += NTHR) {
            const uint32_t en = a.ent[i];
            const int c = (en >> 8) & 255;
            if ((c >> 6) != pq) continue;
            const int r = en & 255, k = (int)(en >> 16);
            float& x = stage[st_idx(c & 63, r)];
            x = fmaf(-gs, a.pt[(r0 + r) * a.K + k], x);
        }
        lds_barrier();
        // G rows: token tl, group g of 8 vocabulary entries; 8 lanes write a token's 64 entries
        // of the pass, one 128-byte line.
#pragma unroll 4
        for (int q = 0; q < kGzRows * kTileM / 8 / NTHR; ++q) {
            const int it = id.tid + NTHR * q;
            const int g = it & 7, tl = it >> 3;
            const int64_t tr = r0 + tl;
            if (tr < a.cc) {
                float x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = stage[st_idx(8 * g + u, tl)];
                store8<T>((T*)a.G + tiled_at<T, kTileM>(tr, n0 + pq * kGzRows + 8 * g, (int64_t)a.n_vt * (kTileN / SW)),
                          x);
            }
        }
        // G^T rows: vocabulary row sr of the pass, group cb of 8 tokens; 32 lanes write a row's
        // 256 tokens.
        if (a.GT) {
#pragma unroll 4
            for (int q = 0; q < kGzRows * kTileM / 8 / NTHR; ++q) {
                const int it = id.tid + NTHR * q;
                const int sr = it >> 5, cb = it & 31;
                const int64_t tr = r0 + cb * 8;
                if (tr < a.ccp) {
                    const float* row = stage + sr * SST;
                    const f32x4 v0 = *(const f32x4*)(row + ((cb * 8) ^ st_swz(sr)));
                    const f32x4 v1 = *(const f32x4*)(row + ((cb * 8 + 4) ^ st_swz(sr)));
                    const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    store8<T>((T*)a.GT + tiled_at<T, kTileM>(n0 + pq * kGzRows + sr, a.gt_col0 + tr, a.ldgt / SW), x);
                }
            }
        }
        lds_barrier();
    };
    f32x4 za[IT], zb[IT];
    load(0, za);
    load(1, zb);
    lds_barrier();  // lse2
    pass(0, za);
    load(2, za);
    pass(1, zb);
    load(3, zb);
    pass(2, za);
    pass(3, zb);
}

// ------------------------------------------------------------------------------------------
// Transpose into a stage-tiled operand with row blocks of 320 (engine.h, kTiled), for the wide
// dH and dW tiles: result row c (c < cols) at K column k0 + r holds src[r*lds + c] for r < rows
// and zero for rows <= r < rows_pad; the result has S stages per row block. 64 x 64 tiles
// through LDS. With dst2 not null the source is also copied, untransposed, into a stage-tiled
// operand with row blocks of 256 and S2 stages (the k_tile_rows layout), from the same loads.

template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int64_t lds, int64_t rows,
                                                   int64_t cols, T* __restrict__ dst, int64_t S, int64_t k0,
                                                   int64_t rows_pad, T* __restrict__ dst2, int64_t S2) {
    // 16-byte global accesses: VEC elements of a source row per load, VEC consecutive rows of
    // one column per store. cols, lds and rows_pad are multiples of VEC and k0 of the stage
    // width, so a vector never leaves its row or its stage. The LDS tile is padded to an odd word
    // stride.
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int LDW = 64 + 4 / (int)sizeof(T);  // row stride in elements: 33 (bf16) or 65 (fp32) words
    constexpr int CPR = 64 / VEC;                 // vectors per tile row
    __shared__ T tile[64][LDW];
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
#pragma unroll
    for (int i = 0; i < 64 * CPR / NTHR; ++i) {
        const int it = threadIdx.x + NTHR * i;
        const int r = it / CPR, cv = (it % CPR) * VEC;
        const int64_t gr = r0 + r, gc = c0 + cv;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gr < rows && gc < cols) v = *(const u32x4*)(src + gr * lds + gc);
        if (dst2 && gr < rows_pad && gc < S2 * 4 * VEC) *(u32x4*)(dst2 + tiled_at<T, kTileM>(gr, gc, S2)) = v;
        const T* e = (const T*)&v;
#pragma unroll
        for (int u = 0; u < VEC; ++u) tile[r][cv + u] = e[u];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 64 * CPR / NTHR; ++i) {
        const int it = threadIdx.x + NTHR * i;
        const int c = it / CPR, rv = (it % CPR) * VEC;
        const int64_t gc = c0 + c, gr = r0 + rv;
        if (gc < cols && gr < rows_pad) {
            u32x4 v;
            T* e = (T*)&v;
#pragma unroll
            for (int u = 0; u < VEC; ++u) e[u] = tile[rv + u][c];
            *(u32x4*)(dst + tiled_at<T, kWideN>(gc, k0 + gr, S)) = v;
        }
    }
}

// Stage-tiled copy (the kTiled operand layout of engine.h) of a row-major src [rows][ld]:
// block (row block b, stage s) holds rows 256b .. 256b+255, columns s*SW .. s*SW+SW-1 (SW = 64
// bytes of elements) as a contiguous [256][SW] array; entries past rows or cols are zero. A
// workgroup writes eight consecutive blocks (128 KB) with consecutive 16-byte stores; its reads
// are 64-byte pieces of 512-byte row segments, the rest of each line read by the same
// workgroup's other blocks.
template <typename T>
__global__ __launch_bounds__(256) void k_tile_rows(const T* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                                                   int64_t S, T* __restrict__ dst) {
    constexpr int VEC = 16 / (int)sizeof(T), SW = 4 * VEC;
    const int64_t rb = blockIdx.y, s0 = (int64_t)blockIdx.x * 8;
    const int nq = (int)min<int64_t>(8, S - s0) * 1024;  // 16-byte chunks to write
    T* out = dst + (rb * S + s0) * (kTileM * SW);
    for (int q = threadIdx.x; q < nq; q += 256) {
        const int sb = q >> 10, r = (q >> 2) & 255, c = q & 3;
        const int64_t gr = rb * kTileM + r, gc = (s0 + sb) * SW + c * VEC;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gr < rows && gc < cols) v = *(const u32x4*)(src + gr * ld + gc);
        *(u32x4*)(out + (int64_t)q * VEC) = v;
    }
}

// ------------------------------------------------------------------------------------------
// dH = G W. The dense path multiplies G [rows][ldg] (vocabulary contiguous) by W [V][d]
// (d contiguous) on 256 x 256 tiles, and so does the fp32 memory-lean backward with its K-blocked
// G_c; the other chunked paths use stage-tiled G_c on 256 x 320 tiles (k_dh_w), with W^T, or
// (the bf16 memory-lean backward) with W as stored.

struct DhArgs {
    const void* G;   // G_c [cc][ldg] row-major or K-blocked [Vp/256][cc][256]; stage-tiled with W^T
    int64_t ldg, Vp;
    const void* W;   // W [V][d], or W^T stage-tiled (row blocks of 320, Vp/SW stages), zero past V
    int64_t d, V;
    int64_t c0, cc;
    int64_t kper;
    int n_split, n_nt, n_mt;
    float* part;
    void* dH;
};

// BLK: G_c is the K-blocked tile of the gradient kernel ([Vp/256][cc][256], the fp32 memory-lean
// backward, which keeps no W^T) instead of row-major [cc][ldg] (the dense path); W is read as
// stored either way.
template <typename T, bool BLK>
__global__ __launch_bounds__(256, 1) void k_dh(DhArgs a) {
    __shared__ u32x4 L[LDS_CHUNKS];
    const WaveId id;
    // Logical tiles are split major, then column tile, then row tile: an XCD's band shares one
    // vocabulary slice of G_c and W.
    const int64_t n_tiles = (int64_t)a.n_split * a.n_nt * a.n_mt;
    const int64_t t = xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles) return;
    const int ks = (int)(t / ((int64_t)a.n_nt * a.n_mt));
    const int rem = (int)(t % ((int64_t)a.n_nt * a.n_mt));
    const int nt = rem / a.n_mt, mt = rem % a.n_mt;
    const int64_t m0 = (int64_t)mt * kTileM, n0 = (int64_t)nt * kTileN;
    const int64_t k_begin = ks * a.kper, k_end = min(a.Vp, k_begin + a.kper);
    f32x16 acc[4][4];
    gemm_tile<T, true, false, BLK>(acc, L, id, (const T*)a.G, BLK ? a.cc : a.ldg, m0, a.cc, k_end, (const T*)a.W,
                                   a.d, n0, a.d, min(a.V, k_end), k_begin, k_end);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = m0 + id.wm * 128 + acc_row(i, e, id.h);
            if (row >= a.cc) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = n0 + id.wn * 128 + j * 32 + id.lr;
                if (col >= a.d) continue;
                const float v = acc[i][j][e];
                if (a.n_split > 1) {
                    a.part[((int64_t)ks * a.cc + row) * a.d + col] = v;
                } else if constexpr (sizeof(T) == 2) {
                    ((bf16_t*)a.dH)[(a.c0 + row) * a.d + col] = (bf16_t)f2bf(v);
                } else {
                    ((float*)a.dH)[(a.c0 + row) * a.d + col] = v;
                }
            }
        }
}

// Same product on 256 x 320 tiles (tokens x hidden) with stage-tiled G_c, and W^T stage-tiled
// (BW = kTiled) or, in the memory-lean backward (bf16), W as stored, whose rows run along V and
// so reach the MFMAs through LDS transpose reads (BW = kTrans).
template <typename T, int BW>
__global__ __launch_bounds__(512, 1) void k_dh_w(DhArgs a) {
    constexpr int SW = 64 / (int)sizeof(T);
    __shared__ u32x4 L[WIDE_LDS_CHUNKS];
    const WaveIdN<8> id;
    const int64_t n_tiles = (int64_t)a.n_split * a.n_nt * a.n_mt;
    const int64_t t = xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles) return;
    const int ks = (int)(t / ((int64_t)a.n_nt * a.n_mt));
    const int rem = (int)(t % ((int64_t)a.n_nt * a.n_mt));
    const int nt = rem / a.n_mt, mt = rem % a.n_mt;
    const int64_t m0 = (int64_t)mt * kTileM, n0 = (int64_t)nt * kWideN;
    const int64_t k_begin = ks * a.kper, k_end = min(a.Vp, k_begin + a.kper);
    f32x4 acc[8][5];
    if constexpr (BW == kTrans)
        gemm_tile_w16<T, kTiled, kTrans>(acc, L, id, (const T*)a.G, a.Vp / SW, m0, a.cc, k_end, (const T*)a.W + n0, a.d,
                                         n0, a.d, min(a.V, k_end), k_begin, k_end);
    else
        gemm_tile_w16<T, kTiled, kTiled>(acc, L, id, (const T*)a.G, a.Vp / SW, m0, a.cc, k_end, (const T*)a.W,
                                         a.Vp / SW, n0, a.d, k_end, k_begin, k_end);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t row = m0 + id.wm * 128 + 16 * i + 4 * (id.lane >> 4) + e;
            if (row >= a.cc) continue;
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int64_t col = n0 + id.wn * 80 + 16 * j + (id.lane & 15);
                if (col >= a.d) continue;
                const float v = acc[i][j][e];
                if (a.n_split > 1) {
                    a.part[((int64_t)ks * a.cc + row) * a.d + col] = v;
                } else if constexpr (sizeof(T) == 2) {
                    ((bf16_t*)a.dH)[(a.c0 + row) * a.d + col] = (bf16_t)f2bf(v);
                } else {
                    ((float*)a.dH)[(a.c0 + row) * a.d + col] = v;
                }
            }
        }
}

template <typename T>
__global__ __launch_bounds__(256) void k_dh_reduce(const float* __restrict__ part, int n_split, int64_t cc,
                                                   int64_t d, int64_t c0, void* __restrict__ dH) {
    const int64_t n4 = cc * d / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        f32x4 s = ((const f32x4*)part)[i];
        for (int k = 1; k < n_split; ++k) s += ((const f32x4*)(part + (int64_t)k * cc * d))[i];
        const int64_t e = i * 4;
        if constexpr (sizeof(T) == 2) {
            uint2 o;
            o.x = f2bf(s[0]) | (f2bf(s[1]) << 16);
            o.y = f2bf(s[2]) | (f2bf(s[3]) << 16);
            *(uint2*)((bf16_t*)dH + c0 * d + e) = o;
        } else {
            *(f32x4*)((float*)dH + c0 * d + e) = s;
        }
    }
}

// ------------------------------------------------------------------------------------------
// dW (+)= G^T H. The dense path reads G [rows][ldg] and H [rows][d] as stored (vocabulary and
// d contiguous) on 256 x 256 tiles; the chunked paths use G_c^T and H_c^T on 256 x 320 tiles
// (k_dw_w).

struct DwArgs {
    // G_c [cc][ldg], G_c K-blocked [Vp/256][cc][256] (g_blk), or G_c^T stage-tiled (row blocks of
    // 256, ldg/SW stages)
    const void* G;
    int64_t ldg, Vp;
    int g_blk;
    const void* H;   // H (rows from c0), or H_c^T stage-tiled (row blocks of 320, ldh/SW stages)
    int64_t ldh;
    int64_t d, V;
    int64_t c0, cc, ccp;
    int accumulate;
    int n_mt, n_nt;
    float* dW;
};

template <typename T>
__global__ __launch_bounds__(256, 1) void k_dw(DwArgs a) {
    constexpr int NT = 256, JN = 4;
    constexpr int IB = 8192 / NT / 2;  // 16-byte items per thread per batch (two batches per pass)
    __shared__ u32x4 L[LDS_CHUNKS];
    const WaveId id;
    // Logical tiles are vocab-row major: an XCD's band shares a few G_c column slabs and H_c.
    const int64_t n_tiles = (int64_t)a.n_mt * a.n_nt;
    const int64_t t = xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles) return;
    const int mt = (int)(t / a.n_nt), nt = (int)(t % a.n_nt);
    const int64_t m0 = (int64_t)mt * kTileM, n0 = (int64_t)nt * kTileN;
    f32x16 acc[4][JN];
    // A K-blocked G_c holds this tile's 256 vocabulary columns as one row-major [cc][256] slab.
    const T* Ga = a.g_blk ? (const T*)a.G + m0 * a.cc : (const T*)a.G;
    gemm_tile<T, false, false>(acc, L, id, Ga, a.g_blk ? (int64_t)kTileN : a.ldg, a.g_blk ? 0 : m0,
                               a.g_blk ? (int64_t)kTileM : a.Vp, a.cc, (const T*)a.H + a.c0 * a.d, a.d, n0, a.d, a.cc,
                               0, a.cc);
    // Read-modify-write through LDS, in two passes of 128 rows. Every dW access is a 16-byte
    // vector and a wave covers 1 KB of one row. The old values of a pass's first half are
    // requested before its staging writes and those of the second half before the first half
    // is added, so the load latency hides behind LDS work.
    const WaveId ie = id.fresh();
    float* stage = (float*)L;
    auto item = [&](int pq, int bt, int k, int& sr, int64_t& row, int64_t& col) {
        const int it = ie.tid + NT * (IB * bt + k);
        sr = it >> 6;
        row = m0 + (sr >> 6) * 128 + pq * 64 + (sr & 63);
        col = n0 + (it & 63) * 4;
    };
    auto load_old = [&](int pq, int bt, f32x4 (&old)[IB]) {
#pragma unroll
        for (int k = 0; k < IB; ++k) {
            int sr;
            int64_t row, col;
            item(pq, bt, k, sr, row, col);
            old[k] = (a.accumulate && row < a.V && col < a.d) ? *(const f32x4*)(a.dW + row * a.d + col)
                                                              : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto add_store = [&](int pq, int bt, const f32x4 (&old)[IB]) {
#pragma unroll
        for (int k = 0; k < IB; ++k) {
            int sr;
            int64_t row, col;
            item(pq, bt, k, sr, row, col);
            if (row < a.V && col < a.d)
                *(f32x4*)(a.dW + row * a.d + col) = old[k] + *(const f32x4*)(stage + st_idx(sr, (int)(col - n0)));
        }
    };
#pragma unroll
    for (int pq = 0; pq < 2; ++pq) {
        f32x4 old0[IB], old1[IB];
        load_old(pq, 0, old0);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int sr = ie.wm * 64 + ii * 32 + blk_row(e, ie.h);
#pragma unroll
                for (int j = 0; j < JN; ++j)
                    stage[st_idx(sr, ie.wn * 128 + j * 32 + ie.lr)] = acc[2 * pq + ii][j][e];
            }
        lds_barrier();
        load_old(pq, 1, old1);
        add_store(pq, 0, old0);
        add_store(pq, 1, old1);
        lds_barrier();
    }
}

// Same product on 256 x 320 tiles (vocabulary x hidden), operands G_c^T and H_c^T (stage-tiled).
// Read-modify-write through LDS in four passes of 64 rows: pass p stages block rows 2p and 2p+1
// of every wave, 32 rows of its 128 (stage row wm*32 + r, tile row wm*128 + 32p + r). Stage rows
// are kWSS floats apart; kWSS % 16 == 4 puts the four row groups a write touches (rows 4 apart)
// on distinct banks. Each thread then handles ten 16-byte items
// per pass, in two batches; old values are requested ahead of the LDS work that hides them.
constexpr int kWSS = 324;

// GL = kTiled: G_c^T and H_c^T stage-tiled over a group of chunks. GL = kTransT (the memory-lean
// backward, bf16): one chunk's stage-tiled G_c and H as stored, both M/N-contiguous for this
// product (their rows run along the tokens), through LDS transpose reads.
template <typename T, int GL>
__global__ __launch_bounds__(512, 1) void k_dw_w(DwArgs a) {
    constexpr int NT = 512, IB = 5;  // items per thread per batch; 2 batches x 512 x 5 = 64 rows x 80
    constexpr int SW = 64 / (int)sizeof(T);
    __shared__ u32x4 L[WIDE_LDS_CHUNKS];
    const WaveIdN<8> id;
    const int64_t n_tiles = (int64_t)a.n_mt * a.n_nt;
    const int64_t t = xcd_tile(blockIdx.x, n_tiles);
    if (t >= n_tiles) return;
    const int mt = (int)(t / a.n_nt), nt = (int)(t % a.n_nt);
    const int64_t m0 = (int64_t)mt * kTileM, n0 = (int64_t)nt * kWideN;
    f32x4 acc[8][5];
    if constexpr (GL == kTransT)
        gemm_tile_w16<T, kTransT, kTrans>(acc, L, id, (const T*)a.G + (m0 / SW) * (kTileM * SW), a.Vp / SW, m0, a.Vp,
                                          a.cc, (const T*)a.H + a.c0 * a.ldh + n0, a.ldh, n0, a.d, a.cc, 0, a.cc);
    else
        gemm_tile_w16<T, kTiled, kTiled>(acc, L, id, (const T*)a.G, a.ldg / SW, m0, a.Vp, a.ccp, (const T*)a.H,
                                         a.ldh / SW, n0, a.d, a.ccp, 0, a.ccp);
    const WaveIdN<8> ie = id.fresh();
    float* stage = (float*)L;
    // dW is addressed through a descriptor at the tile origin with 32-bit offsets (d <= 2^20
    // keeps 256 rows of a tile below 2^31 bytes); items past V or d get an out-of-range offset,
    // which loads zero and drops the store.
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.dW + m0 * a.d + n0);
    const int64_t rows_left = a.V - m0, cols_left = a.d - n0;
    auto item = [&](int p, int bt, int k, int& soff) -> uint32_t {
        const int it = ie.tid + NT * (IB * bt + k);
        const int sr = it / 80, c4 = it % 80;
        const int r = (sr >> 5) * 128 + 32 * p + (sr & 31);
        soff = sr * kWSS + c4 * 4;
        return (r < rows_left && c4 * 4 < cols_left) ? (uint32_t)((r * a.d + c4 * 4) * 4) : kOOB;
    };
    auto load_old = [&](int p, int bt, f32x4 (&old)[IB]) {
#pragma unroll
        for (int k = 0; k < IB; ++k) {
            int soff;
            const uint32_t o = item(p, bt, k, soff);
            old[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0));
        }
    };
    auto add_store = [&](int p, int bt, const f32x4 (&old)[IB]) {
#pragma unroll
        for (int k = 0; k < IB; ++k) {
            int soff;
            const uint32_t o = item(p, bt, k, soff);
            const f32x4 v = old[k] + *(const f32x4*)(stage + soff);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)o, 0, 0);
        }
    };
    const bool acc_old = a.accumulate != 0;
    f32x4 old0[IB], old1[IB];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (acc_old) load_old(p, 0, old0);
        else
#pragma unroll
            for (int k = 0; k < IB; ++k) old0[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sr = ie.wm * 32 + 16 * i2 + 4 * (ie.lane >> 4) + e;
#pragma unroll
                for (int j = 0; j < 5; ++j)
                    stage[sr * kWSS + ie.wn * 80 + 16 * j + (ie.lane & 15)] = acc[2 * p + i2][j][e];
            }
        lds_barrier();
        if (acc_old) load_old(p, 1, old1);
        else
#pragma unroll
            for (int k = 0; k < IB; ++k) old1[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        add_store(p, 0, old0);
        add_store(p, 1, old1);
        lds_barrier();
    }
}

// ------------------------------------------------------------------------------------------
// Dense path.

template <typename T>
__global__ __launch_bounds__(256, 1) void k_dense_logits(const void* H, const void* W, int64_t N, int64_t d,
                                                         int64_t V, float* Z, int64_t ldz) {
    __shared__ u32x4 L[LDS_CHUNKS];
    const WaveId id;
    const int64_t n_rb = (N + kTileM - 1) / kTileM, n_vt = ldz / kTileN;
    const int64_t t = xcd_tile(blockIdx.x, n_rb * n_vt);
    if (t >= n_rb * n_vt) return;
    const int64_t vt = t / n_rb, rb = t % n_rb;
    const int64_t m0 = rb * kTileM, n0 = vt * kTileN;
    f32x16 acc[4][4];
    gemm_tile_kk<T>(acc, L, id, (const T*)H, d, m0, N, d, (const T*)W, d, n0, V, d, 0, d);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = m0 + id.wm * 128 + acc_row(i, e, id.h);
            if (row >= N) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) Z[row * ldz + n0 + id.wn * 128 + j * 32 + id.lr] = acc[i][j][e];
        }
}

__device__ __forceinline__ double block_sum_d(double x, double* red) {
    red[threadIdx.x] = x;
    __syncthreads();
    for (int w = NTHR / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}
__device__ __forceinline__ double block_max_d(double x, double* red) {
    red[threadIdx.x] = x;
    __syncthreads();
    for (int w = NTHR / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// One workgroup per row. Z row: logits (fp32); P row: the dense teacher grid, later G (fp32).
// With a bf16 activation dtype, G is also written as bf16 over the start of the Z row.
__global__ __launch_bounds__(256) void k_dense_rows(float* __restrict__ Z, float* __restrict__ P, int64_t ldz,
                                                    int64_t V, int K, float T, float gsc,
                                                    const int32_t* __restrict__ idx, const void* __restrict__ tlog,
                                                    Dt tdt, const float* __restrict__ grad, float* __restrict__ lse,
                                                    float* __restrict__ row_kl, double* __restrict__ row_sum,
                                                    int g_bf16) {
    __shared__ double red[NTHR];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    float* z = Z + n * ldz;
    float* pg = P + n * ldz;
    const int64_t Vp = ldz;
    // teacher distribution over the K cached entries
    double a = -INFINITY;
    for (int k = tid; k < K; k += NTHR) a = fmax(a, (double)load_t(tlog, tdt, n * K + k) / T);
    const double amax = block_max_d(a, red);
    double ae = 0.0;
    for (int k = tid; k < K; k += NTHR) ae += exp((double)load_t(tlog, tdt, n * K + k) / T - amax);
    const double asum = block_sum_d(ae, red);
    const double alz = amax + log(asum);
    // student log-normaliser over all V
    const double cT = 1.0 / T;
    double mx = -INFINITY;
    for (int64_t v = tid; v < V; v += NTHR) mx = fmax(mx, (double)z[v] * cT);
    mx = block_max_d(mx, red);
    double se = 0.0;
    for (int64_t v = tid; v < V; v += NTHR) se += exp((double)z[v] * cT - mx);
    se = block_sum_d(se, red);
    const double lsed = mx + log(se);
    // expand the cached teacher into the dense grid
    for (int64_t v = tid; v < Vp; v += NTHR) pg[v] = 0.f;
    __syncthreads();
    for (int k = tid; k < K; k += NTHR) {
        const int v = idx[n * K + k];
        if (v >= 0 && v < V) pg[v] = (float)exp((double)load_t(tlog, tdt, n * K + k) / T - alz);  // out-of-range ids are skipped
    }
    __syncthreads();
    // KL over the whole vocabulary (terms with P = 0 contribute 0)
    double kl = 0.0;
    for (int64_t v = tid; v < V; v += NTHR) {
        const float pv = pg[v];
        if (pv > 0.f) kl += (double)pv * (log((double)pv) - ((double)z[v] * cT - lsed));
    }
    kl = block_sum_d(kl, red);
    // gradient grid, in place of the teacher grid
    const float gs = (grad ? grad[0] : 1.f) * gsc;
    const float l2 = (float)(lsed * 1.4426950408889634);
    const float c2 = (float)(cT * 1.4426950408889634);
    for (int64_t v = tid; v < Vp; v += NTHR) pg[v] = v < V ? gs * (exp2_fast(z[v] * c2 - l2) - pg[v]) : 0.f;
    if (g_bf16) {
        __syncthreads();
        bf16_t* gb = (bf16_t*)z;
        for (int64_t v = tid; v < Vp; v += NTHR) gb[v] = (bf16_t)f2bf(pg[v]);
    }
    if (tid == 0) {
        lse[n] = (float)lsed;
        if (row_kl) row_kl[n] = (float)kl;
        row_sum[n] = kl;
    }
}

// ------------------------------------------------------------------------------------------
// Offline top-K cache: per row of teacher logits, the K largest values and their token ids,
// largest first, equal values in lower-id order. Source: "Making knowledge distillation cheap
// enough to run in production" (aiexpert.news), paragraph on the first fix (run the teacher
// once and keep the top-100 tokens per position).
//
// One workgroup per row. Every entry gets a 54-bit key that orders (value desc, id asc):
//   key32 = order-preserving image of the fp32 value (-0 folded onto +0, NaN lowest), and
//   ck = key32 << 22 | (2^22 - 1 - id), unique per entry, larger is better;
// the answer is the K entries with the largest ck. Fast path, two reads of the row:
//   1. each thread keeps the largest value of m interleaved groups of its entries (G = 256 m
//      >= 4K groups in all); the K-th largest group maximum L is a lower bound of the K-th
//      largest value, since the K groups at or above it each hold an entry >= L;
//   2. every entry >= L is collected in LDS (little more than K for logit rows), sorted by ck
//      (bitonic) and the first K written out.
// If more than kTopkSort entries pass the bound (rows full of equal values), a radix select
// takes over: levels of 11 bits histogram the entries matching the prefix fixed so far until
// the bin holding the K-th largest has at most kTopkCap entries, then one more read collects
// everything at or above that bin.

constexpr int kTopkBits = 11, kTopkBins = 1 << kTopkBits;
constexpr int kTopkCap = 2048;   // candidates kept from the threshold bin (radix path)
constexpr int kTopkSort = 4096;  // sort buffer: a power of two >= kTopkCap + kMaxTopK
static_assert(kTopkSort >= kTopkCap + kMaxTopK && (kTopkSort & (kTopkSort - 1)) == 0, "sort buffer");
constexpr int kTopkMaxGroups = 8;  // group maxima per thread (G = 256 m groups, m <= 8)

__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
    if (bits == 0x80000000u) bits = 0u;                     // -0 ranks with +0
    if ((bits & 0x7FFFFFFFu) > 0x7F800000u) return 0u;      // NaN ranks last
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ uint32_t fp32_bits(T x);
template <> __device__ __forceinline__ uint32_t fp32_bits<bf16_t>(bf16_t x) { return (uint32_t)x << 16; }
template <> __device__ __forceinline__ uint32_t fp32_bits<float>(float x) { return __float_as_uint(x); }

// Largest of the entries of a 16-byte chunk, as fp32 (a NaN entry is ignored unless all are NaN).
template <typename T>
__device__ __forceinline__ float chunk_max(const u32x4& c) {
    if constexpr (sizeof(T) == 2) {
        const float a = fmaxf(__uint_as_float(c[0] << 16), __uint_as_float(c[0] & 0xFFFF0000u));
        const float b = fmaxf(__uint_as_float(c[1] << 16), __uint_as_float(c[1] & 0xFFFF0000u));
        const float e = fmaxf(__uint_as_float(c[2] << 16), __uint_as_float(c[2] & 0xFFFF0000u));
        const float f = fmaxf(__uint_as_float(c[3] << 16), __uint_as_float(c[3] & 0xFFFF0000u));
        return fmaxf(fmaxf(a, b), fmaxf(e, f));
    } else {
        return fmaxf(fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1])),
                     fmaxf(__uint_as_float(c[2]), __uint_as_float(c[3])));
    }
}

struct KeepAll {
    __device__ __forceinline__ bool operator()(float) const { return true; }
};

// Calls f(v, bits) for every entry of row x[0..V) handled by this thread, with 16-byte loads
// for the aligned body; j counts this thread's loads (for the group choice). With a `keep`
// test, the entries of a body chunk are visited only if keep(largest entry of the chunk) holds:
// a caller that wants the entries >= L skips whole chunks below L with one comparison.
template <typename T, typename F, typename Keep = KeepAll>
__device__ __forceinline__ void topk_scan(const T* x, int V, F&& f, Keep keep = Keep()) {
    constexpr int VEC = 16 / sizeof(T);
    const int tid = threadIdx.x;
    const int head = (int)(((16 - ((uintptr_t)x & 15)) & 15) / sizeof(T));
    const int h = head < V ? head : V;
    if (tid < h) f(tid, fp32_bits<T>(x[tid]), 0);
    const int nvec = (V - h) / VEC;
    const u32x4* xv = (const u32x4*)(x + h);
    auto each = [&](const u32x4& c, int q, int j) {
        if (!keep(chunk_max<T>(c))) return;
        const int v0 = h + q * VEC;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f(v0 + 2 * u, c[u] << 16, j);
                f(v0 + 2 * u + 1, c[u] & 0xFFFF0000u, j);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) f(v0 + u, c[u], j);
        }
    };
    // eight 16-byte loads in flight per lane
    int j = 0;
    int q = tid;
    for (; q + 7 * NTHR < nvec; q += 8 * NTHR, j += 8) {
        u32x4 c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = xv[q + u * NTHR];
#pragma unroll
        for (int u = 0; u < 8; ++u) each(c[u], q + u * NTHR, j + u);
    }
    for (; q < nvec; q += NTHR, ++j) each(xv[q], q, j);
    for (int v = h + nvec * VEC + tid; v < V; v += NTHR) f(v, fp32_bits<T>(x[v]), 0);
}

// Largest value of each of M interleaved groups of this thread's entries (load j of the thread
// goes to group j % M), eight 16-byte loads in flight per lane. M is a power of two up to 8, so
// within a batch of eight loads the group of each is known at compile time.
template <typename T, int M>
__device__ __forceinline__ void topk_scan_max(const T* x, int V, float (&gmax)[kTopkMaxGroups]) {
    constexpr int VEC = 16 / sizeof(T);
    const int tid = threadIdx.x;
    const int head = (int)(((16 - ((uintptr_t)x & 15)) & 15) / sizeof(T));
    const int h = head < V ? head : V;
    if (tid < h) gmax[0] = fmaxf(gmax[0], __uint_as_float(fp32_bits<T>(x[tid])));
    const int nvec = (V - h) / VEC;
    const u32x4* xv = (const u32x4*)(x + h);
    int j = 0;
    int q = tid;
    for (; q + 7 * NTHR < nvec; q += 8 * NTHR, j += 8) {
        u32x4 c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = xv[q + u * NTHR];
#pragma unroll
        for (int u = 0; u < 8; ++u) gmax[u % M] = fmaxf(gmax[u % M], chunk_max<T>(c[u]));
    }
    for (; q < nvec; q += NTHR, ++j) {
        const float r = chunk_max<T>(xv[q]);
        const int g = j & (M - 1);
#pragma unroll
        for (int t = 0; t < M; ++t)
            if (t == g) gmax[t] = fmaxf(gmax[t], r);
    }
    for (int v = h + nvec * VEC + tid; v < V; v += NTHR) gmax[0] = fmaxf(gmax[0], __uint_as_float(fp32_bits<T>(x[v])));
}

__device__ __forceinline__ uint64_t topk_ck(int v, uint32_t bits) {
    return ((uint64_t)order_key(bits) << 22) | (uint64_t)(0x3FFFFF - v);
}

// Bitonic sort of a[0..P) descending (P a power of two), by all NT threads of the block. With
// LDS_ONLY the steps are separated by barriers that wait for this wave's LDS operations only, so
// global loads issued before the sort stay in flight through it.
template <int NT = NTHR, bool LDS_ONLY = false>
__device__ __forceinline__ void bitonic_desc(uint64_t* a, int P) {
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += NT) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a0 = a[lo], a1 = a[hi];
                if ((a0 < a1) == desc) {
                    a[lo] = a1;
                    a[hi] = a0;
                }
            }
            if constexpr (LDS_ONLY)
                lds_barrier();
            else
                __syncthreads();
        }
    }
}

// Bitonic sort of a[0..P) descending (P a power of two) by one wave, with no barriers: the LDS
// runs one wave's accesses in issue order, so each step sees the previous step's writes.
__device__ __forceinline__ void wave_bitonic_desc(uint64_t* a, int P) {
    const int lane = threadIdx.x & 63;
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = lane; i < P / 2; i += 64) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a0 = a[lo], a1 = a[hi];
                const bool swap = (a0 < a1) == desc;
                a[lo] = swap ? a1 : a0;
                a[hi] = swap ? a0 : a1;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// With only_flagged, a workgroup handles its row only if k_topk_reg left the row's first id at
// -1 (the rows whose register-held bound did not settle them); the others keep their output.
template <typename T>
__global__ __launch_bounds__(256) void k_topk(const T* __restrict__ X, int64_t ld, int64_t N, int V, int K,
                                              int32_t* __restrict__ idx_out, T* __restrict__ val_out,
                                              int only_flagged) {
    __shared__ uint32_t hist[2][kTopkBins];  // two copies (waves 0, 2 and 1, 3): 49 KB of LDS, three rows per CU
    __shared__ uint64_t cand[kTopkSort];
    __shared__ uint32_t wsum[NTHR];
    __shared__ int s_bin, s_above, s_cnt, s_ncoll;
    const int tid = threadIdx.x, w = tid >> 6;
    const int64_t n = blockIdx.x;
    if (only_flagged && idx_out[n * K] != -1) return;
    const T* x = X + n * ld;
    int nc = 0;
    bool done = false;

    // ---- fast path: lower bound from group maxima, then one collecting read. Both reads
    // work on fp32 values (max and compare treat -0 as +0, as the key does); only the
    // collected entries get their 54-bit keys.
    {
        int m = 1;  // groups per thread: the power of two with 256 m >= 4K, at most 8
        while (m < kTopkMaxGroups && NTHR * m < 4 * K) m <<= 1;
        float gmax[kTopkMaxGroups];
#pragma unroll
        for (int g = 0; g < kTopkMaxGroups; ++g) gmax[g] = -INFINITY;
        switch (m) {
            case 1: topk_scan_max<T, 1>(x, V, gmax); break;
            case 2: topk_scan_max<T, 2>(x, V, gmax); break;
            case 4: topk_scan_max<T, 4>(x, V, gmax); break;
            default: topk_scan_max<T, 8>(x, V, gmax); break;
        }
        const int G = NTHR * m;  // <= 2048 <= kTopkSort
        int P = 1;
        while (P < G) P <<= 1;
#pragma unroll
        for (int q = 0; q < kTopkMaxGroups; ++q)
            if (q < m) cand[q * NTHR + tid] = (uint64_t)order_key(__float_as_uint(gmax[q]));
        for (int i = G + tid; i < P; i += NTHR) cand[i] = 0ull;
        __syncthreads();
        bitonic_desc(cand, P);
        const uint32_t Lk = (uint32_t)cand[K - 1];
        // back to the value: keys >= 2^31 are non-negative floats
        const float L = __uint_as_float(Lk & 0x80000000u ? (Lk & 0x7FFFFFFFu) : ~Lk);
        if (tid == 0) s_ncoll = 0;
        __syncthreads();
        topk_scan<T>(
            x, V,
            [&](int v, uint32_t bits, int) {
                if (__uint_as_float(bits) >= L) {
                    const int pos = atomicAdd(&s_ncoll, 1);
                    if (pos < kTopkSort) cand[pos] = topk_ck(v, bits);
                }
            },
            [L](float mx) { return mx >= L; });
        __syncthreads();
        nc = s_ncoll;
        done = nc >= K && nc <= kTopkSort;  // fewer than K only if NaNs were skipped
        __syncthreads();
    }

    // ---- radix select when too many entries passed the bound
    if (!done) {
        uint64_t prefix = 0;
        int shift = 54, need = K;
        while (true) {
            const int wd = shift < kTopkBits ? shift : kTopkBits;
            const int s = shift - wd;
            for (int i = tid; i < 2 * kTopkBins; i += NTHR) (&hist[0][0])[i] = 0u;
            __syncthreads();
            topk_scan<T>(x, V, [&](int v, uint32_t bits, int) {
                const uint64_t ck = topk_ck(v, bits);
                if ((ck >> shift) == prefix) atomicAdd(&hist[w & 1][(uint32_t)(ck >> s) & ((1u << wd) - 1u)], 1u);
            });
            __syncthreads();
            // Bins of this level, highest first: thread t owns bins [8t, 8t+8) counted from the top.
            constexpr int PER = kTopkBins / NTHR;
            uint32_t mine[PER], tot = 0;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int b = kTopkBins - 1 - (tid * PER + q);
                mine[q] = hist[0][b] + hist[1][b];
                tot += mine[q];
            }
            wsum[tid] = tot;
            __syncthreads();
            if (tid == 0) {  // exclusive scan of the 256 thread totals, from the top
                uint32_t run = 0;
                for (int t = 0; t < NTHR; ++t) {
                    const uint32_t c = wsum[t];
                    wsum[t] = run;
                    run += c;
                }
            }
            __syncthreads();
            uint32_t above = wsum[tid];
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                if (above < (uint32_t)need && above + mine[q] >= (uint32_t)need) {
                    s_bin = kTopkBins - 1 - (tid * PER + q);
                    s_above = (int)above;
                    s_cnt = (int)mine[q];
                }
                above += mine[q];
            }
            __syncthreads();
            prefix = (prefix << wd) | (uint64_t)s_bin;
            need -= s_above;
            shift = s;
            const int cnt = s_cnt;
            __syncthreads();
            if (cnt <= kTopkCap || shift == 0) break;
        }
        // Every entry at or above the threshold bin: K - need above it, the bin's own after.
        if (tid == 0) s_ncoll = 0;
        __syncthreads();
        topk_scan<T>(x, V, [&](int v, uint32_t bits, int) {
            const uint64_t ck = topk_ck(v, bits);
            if ((ck >> shift) >= prefix) cand[atomicAdd(&s_ncoll, 1)] = ck;
        });
        __syncthreads();
        nc = s_ncoll;
    }

    int P = 1;
    while (P < nc) P <<= 1;
    for (int i = nc + tid; i < P; i += NTHR) cand[i] = 0ull;  // below every real key
    __syncthreads();
    bitonic_desc(cand, P);
    for (int k = tid; k < K; k += NTHR) {
        const int v = 0x3FFFFF - (int)(cand[k] & 0x3FFFFFull);
        idx_out[n * K + k] = v;
        val_out[n * K + k] = x[v];
    }
}

// One read of each row: a persistent grid, one workgroup of kTkrThreads per CU, holds a whole row
// on chip. Thread t owns the 16-byte chunks t, t + 512, ... of the row, up to kTkrChunks of them
// (204,800 bf16 or 102,400 fp32 entries); the last kTkrLds of its slots are loaded straight into
// LDS, the others into registers. Per row:
//   1. as the chunks land, each one's largest entry goes to LDS and into the thread's largest
//      entry. Each wave finds the t-th largest of its 64 thread maxima, t = ceil(K / 8), and the
//      bound L is the least of the 8 waves' values. Every wave has t threads whose largest entry
//      is >= its value >= L, so at least 8 t >= K entries of the row are >= L: L bounds the K-th
//      largest value from below;
//   2. the chunks whose largest entry is >= L are copied to an LDS list, and the block takes the
//      list apart into the candidates, the entries >= L (all of the row's top K among them);
//   3. the next row's loads are issued into the same registers and LDS slots, and while they are
//      in flight each candidate counts the candidates with a larger key. That count is its place
//      in the output, which it writes if the count is below K.
// Appends to the LDS lists take their places from a prefix count over the wave and one atomic
// per wave. A row with fewer than K candidates (NaN), more than the buffers hold (many equal
// values) or a bound of -inf is left with its first id at -1; k_topk then redoes those rows
// exactly.
constexpr int kTkrThreads = 512, kTkrChunks = 50, kTkrCand = 1024, kTkrList = 1024, kTkrMaxK = 128;
constexpr int kTkrLds = 8;  // slots loaded into LDS
constexpr int kNonTemporal = 2;  // cache-policy operand of a buffer load: non-temporal

// The pass's sort key: the 54-bit order (value, then lower id first) moved up one bit, and a last
// bit that marks a -0 entry, which the order ranks with +0. Keys stay distinct and ordered as
// before, and the stored value can be rebuilt from the key.
__device__ __forceinline__ uint64_t tkr_key(int v, uint32_t bits) {
    return (topk_ck(v, bits) << 1) | (uint64_t)(bits == 0x80000000u);
}

// Exclusive prefix sum over the wave of a count below 2^NB, and the wave's total, from one ballot
// per bit (all lanes active).
template <int NB>
__device__ __forceinline__ int wave_prefix(int cnt, int& total) {
    int pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint64_t m = __ballot((cnt >> b) & 1);
        pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
        tot += __popcll(m) << b;
    }
    total = tot;
    return pre;
}

template <typename T>
__global__ __launch_bounds__(kTkrThreads, 1) void k_topk_reg(const T* __restrict__ X, int64_t ld, int64_t N, int V,
                                                             int K, int32_t* __restrict__ idx_out,
                                                             T* __restrict__ val_out) {
    constexpr int NT = kTkrThreads, VEC = 16 / (int)sizeof(T), NW = NT / 64, S = kTkrChunks;
    constexpr int NL = kTkrLds, NR = S - NL;  // slots in LDS, in registers
    // A chunk's largest entry is kept as a bf16 value: exactly for bf16 rows, rounded up for fp32
    // rows (the test against the bound then lets through a few more chunks, whose entries are
    // compared exactly). Eight go to a 16-byte LDS vector, thread-major, so that a thread writes
    // and reads its own with a few wide accesses.
    constexpr int CPV = 8, CMV = (S + CPV - 1) / CPV;
    __shared__ u32x4 lslot[NL * NT];  // slots NR .. S-1, slot-major
    __shared__ u32x4 cmv[NT * CMV];   // chunk maxima
    __shared__ uint64_t cand[kTkrCand];
    __shared__ u32x4 chl[kTkrList];   // chunks holding an entry >= the bound
    __shared__ int chq[kTkrList];     // and their positions in the row (in chunks)
    __shared__ uint32_t wkey[NW];
    __shared__ int s_n[2], s_nch[2];  // list lengths; rows alternate between the two pairs
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nvec = V / VEC, tail = V - nvec * VEC;  // row bases are 16-byte aligned (host check)
    constexpr int kFull = 16;  // slots below this hold row entries in every thread (host check:
                               // nvec >= kTkrChunks * NT / 3)
    const int t_w = (K + NW - 1) / NW;  // <= 64 since K <= kTkrMaxK
    // Every slot is loaded: a slot past the row's end reads the row's last chunk again and counts
    // as -inf. Below kFull the slot offset goes in the scalar operand; above, the whole offset is
    // clamped in the lane's. Each load is issued as soon as its offset exists, marked
    // non-temporal (the row is read once; streaming reads ran about 3 % faster so). Values derived
    // from the thread index are recomputed for each row from an opaque copy of it: held across
    // rows they would take registers the row needs.
    u32x4 c[NR];
    T traw;  // an entry of the row's tail (past the last whole chunk): this thread's if it has one
    auto load = [&](int64_t r) {
        const T* x = X + r * ld;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(x);
        int o = tid * 16, sb = 0, last = (nvec - 1) * 16, wb = __builtin_amdgcn_readfirstlane(w) * 64;
        asm volatile("" : "+v"(o), "+s"(sb), "+s"(last), "+s"(wb));
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int so = j < kFull ? sb + j * NT * 16 : sb;
            const int vo = j < kFull ? o : min(o + j * NT * 16, last);
            if (j < NR)
                c[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, kNonTemporal));
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lslot + (j - NR) * NT + wb), 16, vo, so, 0,
                                                         kNonTemporal);
            __builtin_amdgcn_sched_barrier(0);
        }
        // unconditional and in bounds, so that nothing waits for it before the chunks are used
        int ti = tid;
        asm volatile("" : "+v"(ti));
        traw = x[tail > 0 ? nvec * VEC + min(ti, tail - 1) : 0];
    };
    if (tid < 2) s_n[tid] = 0, s_nch[tid] = 0;
    int64_t r = blockIdx.x;
    int par = 0;
    if (r < N) load(r);
    while (r < N) {
        // 1. chunk maxima and the thread's largest entry (NaN ignored)
        float mx = -INFINITY;
        uint32_t tb;  // this thread's tail entry, or -inf
        {
            int tq = tid;
            asm volatile("" : "+v"(tq));
            uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < S; ++j) {
                if (j == NR) wait_vmem();  // the LDS slots, loaded last, have landed (a lane reads its own)
                float cm = chunk_max<T>(j < NR ? c[j < NR ? j : 0] : lslot[(j - NR) * NT + tq]);
                if (j >= kFull && tq + j * NT >= nvec) cm = -INFINITY;
                mx = fmaxf(mx, cm);
                const int e = j % CPV;
                const uint32_t cb = __float_as_uint(cm);
                uint32_t h = cb >> 16;
                if constexpr (sizeof(T) == 4) h += (cb < 0x7F800000u && (cb & 0xFFFFu) != 0u) ? 1u : 0u;
                pk[e / 2] = (e & 1) ? (pk[e / 2] | (h << 16)) : h;
                if (e == CPV - 1 || j == S - 1) cmv[tq * CMV + j / CPV] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            }
            tb = tq < tail ? fp32_bits<T>(traw) : 0xFF800000u;
            mx = fmaxf(mx, __uint_as_float(tb));
        }
        // The wave's t-th largest key, bit by bit from the top: a bit is set if at least `need`
        // lanes match the prefix with it set. bf16 values fill the top 16 bits of the key; the
        // rest then follows from the sign (0 for non-negative values, all ones for negative).
        const uint32_t key = order_key(__float_as_uint(mx));
        uint32_t kw = 0;
        {
            int need = t_w;
            constexpr int LOW = sizeof(T) == 2 ? 16 : 0;
#pragma unroll
            for (int b = 31; b >= LOW; --b) {
                const uint32_t want = (kw >> b) | 1u;
                const int cnt = __popcll(__ballot((key >> b) == want));
                if (cnt >= need)
                    kw |= 1u << b;
                else
                    need -= cnt;
            }
            if constexpr (LOW > 0) kw |= (kw & 0x80000000u) ? 0u : 0xFFFFu;
        }
        if (lane == 0) wkey[w] = kw;
        lds_barrier();
        if (tid == 0) s_n[par ^ 1] = 0, s_nch[par ^ 1] = 0;  // the next row's; the last row read them
        uint32_t lk = wkey[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) lk = min(lk, wkey[i]);
        // back to the value: keys >= 2^31 are non-negative floats (mx is never NaN, so lk > 0).
        // A bound of -inf would take in the padding slots: such a row is left to k_topk.
        const bool ok_bound = lk > 0x007FFFFFu;
        const float L = ok_bound ? __uint_as_float(lk & 0x80000000u ? (lk & 0x7FFFFFFFu) : ~lk) : INFINITY;
        // 2. chunks with an entry >= L to the list (NaN compares false) ...
        {
            int qb = tid;
            asm volatile("" : "+v"(qb));
            // Both passes read the maxima from LDS: held between them they would take registers
            // the row needs.
            auto passes = [&](const u32x4& mv, int j) {
                const int e = j % CPV;
                const uint32_t word = mv[e / 2];
                return __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16)) >= L;
            };
            int cnt = 0;
#pragma unroll
            for (int v = 0; v < CMV; ++v) {
                const u32x4 mv = cmv[qb * CMV + v];
#pragma unroll
                for (int j = v * CPV; j < min((v + 1) * CPV, S); ++j) cnt += passes(mv, j) ? 1 : 0;
            }
            asm volatile("" ::: "memory");
            int total;
            int pos = wave_prefix<6>(cnt, total);
            int base = 0;
            if (lane == 0 && total > 0) base = atomicAdd(&s_nch[par], total);
            pos += __builtin_amdgcn_readfirstlane(base);
            // past the list's end every chunk lands on its last entry: the row then goes to k_topk
#pragma unroll
            for (int j = 0; j < S; ++j) {
                const u32x4 mv = cmv[qb * CMV + j / CPV];
                if (passes(mv, j)) {
                    const int at = min(pos, kTkrList - 1);
                    chl[at] = j < NR ? c[j < NR ? j : 0] : lslot[(j - NR) * NT + qb];
                    chq[at] = qb + j * NT;
                    ++pos;
                }
            }
            if (qb < tail && __uint_as_float(tb) >= L) {
                const int p = atomicAdd(&s_n[par], 1);  // at most 7 lanes, before any other append
                cand[p] = tkr_key(nvec * VEC + qb, tb);
            }
        }
        lds_barrier();
        // ... and its entries >= L to the candidates (after the tail entries already there)
        const int nch = s_nch[par];
        for (int i0 = 0; i0 < min(nch, kTkrList); i0 += NT) {
            const int i = i0 + tid;
            uint32_t bits[VEC];
            uint32_t em = 0;
            int q = 0;
            if (i < min(nch, kTkrList)) {
                const u32x4 ch = chl[i];
                q = chq[i];
#pragma unroll
                for (int u = 0; u < VEC; ++u) {
                    bits[u] = sizeof(T) == 2 ? ((u & 1) ? (ch[u / 2] & 0xFFFF0000u) : (ch[u / 2] << 16)) : ch[u];
                    em |= (uint32_t)(__uint_as_float(bits[u]) >= L) << u;
                }
            }
            int total;
            int pos = wave_prefix<4>(__popc(em), total);
            int base = 0;
            if (lane == 0 && total > 0) base = atomicAdd(&s_n[par], total);
            pos += __builtin_amdgcn_readfirstlane(base);
#pragma unroll
            for (int u = 0; u < VEC; ++u) {
                if ((em >> u) & 1) {
                    if (pos < kTkrCand) cand[pos] = tkr_key(q * VEC + u, bits[u]);
                    ++pos;
                }
            }
        }
        lds_barrier();
        const int nc = s_n[par];
        // 3. The registers and LDS slots are free: the next row's loads go out, then each wave
        // places its candidates with no barrier (a wave waits at load issue while the CU's memory
        // queue is full; work shared through barriers would wait for every wave's loads to be
        // requested). A candidate's place is the number of candidates with a larger key. The
        // next row's first barrier orders the reuse of the LDS lists and counters.
        const int64_t rn = r + gridDim.x;
        if (rn < N) load(rn);
        if (!ok_bound || nc < K || nc > kTkrCand || nch > kTkrList) {
            if (tid == 0) idx_out[r * K] = -1;  // left to k_topk
        } else {
            for (int i = tid; i < nc; i += NT) {
                const uint64_t me = cand[i];
                int rank = 0;
                int j = 0;
                for (; j + 2 <= nc; j += 2) {
                    const uint64_t a0 = cand[j], a1 = cand[j + 1];
                    rank += (int)(a0 > me) + (int)(a1 > me);
                }
                if (j < nc) rank += (int)(cand[j] > me);
                if (rank < K) {
                    const uint32_t ok = (uint32_t)(me >> 23);
                    const uint32_t bits = (me & 1ull) ? 0x80000000u : (ok & 0x80000000u ? ok & 0x7FFFFFFFu : ~ok);
                    idx_out[r * K + rank] = 0x3FFFFF - (int)((me >> 1) & 0x3FFFFFull);
                    if constexpr (sizeof(T) == 2)
                        val_out[r * K + rank] = (bf16_t)(bits >> 16);
                    else
                        val_out[r * K + rank] = __uint_as_float(bits);
                }
            }
        }
        par ^= 1;
        r = rn;
    }
}


// ------------------------------------------------------------------------------------------
// Launchers.

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Waves per workgroup of the dW and dH GEMMs: eight (two per SIMD) hide more of the operand
// latency than four.
constexpr int kGradWaves = 8, kFwdWaves = 8;

// Vocab lanes of the forward: at least 8, and enough units to give every CU one.
// Vocabulary lanes Q of the persistent forward: unit (row block, lane q) walks vocab tiles q,
// q + Q, ... The grid's workgroup w takes units w, w + P, w + 2P, ... of its XCD band, so the
// busiest workgroup does ceil(units / P) units of up to ceil(n_vt / Q) tiles. Among Q in
// 4..16 pick the one with the least of that, preferring Q near 8 (4 row blocks x 8 lanes per
// XCD share operands in L2 best); at least 256 units when the rows are few.
int fwd_vsplits(int64_t N, int64_t V) {
    const int64_t n_rb = (N + kTileM - 1) / kTileM;
    const int64_t n_vt = (V + kTileN - 1) / kTileN;
    const int64_t q_min = std::max<int64_t>(4, (256 + n_rb - 1) / n_rb);
    if (q_min >= n_vt) return (int)n_vt;
    const int64_t P = 256;
    int64_t best_q = std::min<int64_t>(std::max<int64_t>(8, q_min), n_vt), best = INT64_MAX;
    for (int64_t q = q_min; q <= std::min<int64_t>(16, n_vt); ++q) {
        const int64_t load = ((n_rb * q + P - 1) / P) * ((n_vt + q - 1) / q);
        const int64_t dist = q > 8 ? q - 8 : 8 - q;
        const int64_t best_dist = best_q > 8 ? best_q - 8 : 8 - best_q;
        if (load < best || (load == best && dist < best_dist)) {
            best = load;
            best_q = q;
        }
    }
    return (int)best_q;
}

// Compute units of the current device (cached per device id).
static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

static unsigned grid_xcd(int64_t n_tiles) { return (unsigned)(8 * ((n_tiles + 7) / 8)); }

int dh_splits(int64_t cc, int64_t d, int64_t V, bool wide) {
    const int64_t tiles = ((cc + kTileM - 1) / kTileM) * ((d + (wide ? kWideN : kTileN) - 1) / (wide ? kWideN : kTileN));
    if (tiles >= 512) return 1;
    const int64_t ksteps = (V + 63) / 64;
    const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(32, ksteps / 4));
    if (!wide) {
        const int64_t s = std::min<int64_t>((768 + tiles - 1) / tiles, s_max);
        return (int)std::max<int64_t>(s, 1);
    }
    // Fewest splits that fill the 256 compute units in whole rounds to within 5 % (each split
    // adds a partial of cc x d floats to write and reduce); else the best fill up to 3 rounds.
    int64_t best = 1;
    double best_fill = 0.0;
    for (int64_t s = 1; s <= s_max; ++s) {
        const int64_t n = tiles * s;
        const double fill = (double)n / (double)(((n + 255) / 256) * 256);
        if (n >= 256 && fill >= 0.95) return (int)s;
        if (n <= 768 && fill > best_fill + 1e-9) {
            best = s;
            best_fill = fill;
        }
    }
    return (int)best;
}

int combine_blocks(int64_t N) { return (int)((N + kCombRows - 1) / kCombRows); }

hipError_t launch_plan(const int32_t* idx, int64_t row0, int64_t row1, int64_t K, int64_t V, int32_t* off,
                       uint32_t* ent, hipStream_t s) {
    const int n_rb = (int)((row1 - row0 + kTileM - 1) / kTileM);
    const int n_vt = (int)((V + kTileN - 1) / kTileN);
    KD_LAUNCH(kKindPlan, s, k_plan, dim3(n_rb), dim3(kPlanThreads), 0, s, idx, row0, row1, (int)K, V, n_vt, off, ent);
    return hipGetLastError();
}

hipError_t launch_teacher_prob(const void* tlog, Dt tdt, int64_t row0, int64_t row1, int64_t K, float T,
                               float* pt, hipStream_t s) {
    const int64_t rows = row1 - row0;
    KD_LAUNCH(kKindTeacherProb, s, k_teacher_prob, dim3((unsigned)((rows + 3) / 4)), dim3(NTHR), 0, s, tlog, tdt, row0, row1,
                       (int)K, T, pt);
    return hipGetLastError();
}

hipError_t launch_validate(const int32_t* idx, int64_t N, int64_t K, int64_t V, uint32_t* status, hipStream_t s) {
    KD_LAUNCH(kKindValidate, s, k_zero_u32, dim3(1), dim3(64), 0, s, status, 1);
    KD_LAUNCH(kKindValidate, s, k_validate, dim3((unsigned)((N + 3) / 4)), dim3(NTHR), 0, s, idx, N, (int)K, V, status);
    return hipGetLastError();
}

hipError_t launch_fwd(const Shape& sh, const void* H, const void* W, const int32_t* plan_off,
                      const uint32_t* plan_ent, int n_vsplit, float2* part, float* zk, float* zt, int64_t ldzt,
                      hipStream_t s, int64_t tiled_S) {
    FwdArgs a;
    a.H = H;
    a.W = W;
    a.ldh = a.ldw = tiled_S > 0 ? tiled_S : sh.d;
    a.N = sh.N;
    a.d = sh.d;
    a.V = sh.V;
    a.K = sh.K;
    a.c = kLog2e / sh.T;
    a.off = plan_off;
    a.ent = plan_ent;
    a.n_vt = (int)((sh.V + kTileN - 1) / kTileN);
    a.Q = n_vsplit;
    a.n_unit = ((sh.N + kTileM - 1) / kTileM) * (int64_t)n_vsplit;
    a.part = part;
    a.zk = zk;
    a.zt = zt;
    a.ldzt = ldzt;
    // One workgroup per CU (the LDS use allows no more), a multiple of 8 for the XCD bands.
    const int64_t cus = std::max(8, device_cus() / 8 * 8);
    const unsigned grid = (unsigned)std::min<int64_t>(cus, 8 * ((a.n_unit + 7) / 8));
    const dim3 blk(64 * kFwdWaves);
    const bool t = tiled_S > 0;
    if (sh.act == Dt::BF16) {
        if (zt && t)
            KD_LAUNCH(kKindFwd, s, (k_fwd<bf16_t, true, kFwdWaves, kTiled>), dim3(grid), blk, 0, s, a);
        else if (zt)
            KD_LAUNCH(kKindFwd, s, (k_fwd<bf16_t, true, kFwdWaves, kRow>), dim3(grid), blk, 0, s, a);
        else if (t)
            KD_LAUNCH(kKindFwd, s, (k_fwd<bf16_t, false, kFwdWaves, kTiled>), dim3(grid), blk, 0, s, a);
        else
            KD_LAUNCH(kKindFwd, s, (k_fwd<bf16_t, false, kFwdWaves, kRow>), dim3(grid), blk, 0, s, a);
    } else {
        if (zt && t)
            KD_LAUNCH(kKindFwd, s, (k_fwd<float, true, kFwdWaves, kTiled>), dim3(grid), blk, 0, s, a);
        else if (zt)
            KD_LAUNCH(kKindFwd, s, (k_fwd<float, true, kFwdWaves, kRow>), dim3(grid), blk, 0, s, a);
        else if (t)
            KD_LAUNCH(kKindFwd, s, (k_fwd<float, false, kFwdWaves, kTiled>), dim3(grid), blk, 0, s, a);
        else
            KD_LAUNCH(kKindFwd, s, (k_fwd<float, false, kFwdWaves, kRow>), dim3(grid), blk, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const Shape& sh, const float2* part, int n_part, const float* zk, const void* tlog,
                          float* lse, float* row_kl, double* blk_sum, int* n_blk_out, hipStream_t s) {
    const int nb = combine_blocks(sh.N);
    KD_LAUNCH(kKindCombine, s, k_combine, dim3(nb), dim3(NTHR), 0, s, part, n_part, sh.N, (int)sh.K, sh.T, zk, tlog, sh.tlog,
                       lse, row_kl, blk_sum);
    if (n_blk_out) *n_blk_out = nb;
    return hipGetLastError();
}

hipError_t launch_loss_final(const Shape& sh, const double* blk_sum, int n_blk, float* loss, hipStream_t s) {
    const double scale = (double)sh.T * (double)sh.T / (double)sh.n_norm;
    KD_LAUNCH(kKindLossFinal, s, k_loss_final, dim3(1), dim3(NTHR), 0, s, blk_sum, n_blk, scale, loss);
    return hipGetLastError();
}

hipError_t launch_bwd_grad(const Shape& sh, const void* H, const void* W, const float* lse, const float* pt,
                           const float* grad_loss, int64_t c0, int64_t cc, const int32_t* plan_off,
                           const uint32_t* plan_ent, void* Gc, bool g_tiled, void* GT, int64_t ldgt, int64_t gt_col0,
                           hipStream_t s, int64_t tiled_S) {
    GradArgs a;
    a.H = H;
    a.W = W;
    a.ldh = a.ldw = tiled_S > 0 ? tiled_S : sh.d;
    a.zt = nullptr;
    a.ldzt = a.zt_col0 = 0;
    a.d = sh.d;
    a.V = sh.V;
    a.K = sh.K;
    a.c = kLog2e / sh.T;
    a.gsc = sh.T / sh.n_norm;
    a.grad = grad_loss;
    a.lse = lse;
    a.pt = pt;
    a.c0 = c0;
    a.cc = cc;
    a.off = plan_off;
    a.ent = plan_ent;
    a.n_vt = (int)((sh.V + kTileN - 1) / kTileN);
    a.n_rbc = (int)((cc + kTileM - 1) / kTileM);
    a.G = Gc;
    a.GT = GT;
    a.ldgt = ldgt;
    a.gt_col0 = gt_col0;
    a.ccp = round_up(cc, 32);
    if (GT && (ldgt % 32 != 0 || gt_col0 % 32 != 0)) return hipErrorInvalidValue;
    // One tile per workgroup: measured a little faster than the persistent launch, whose
    // workgroups stay in lockstep and so issue their tile stores all at once.
    const dim3 grid(grid_xcd((int64_t)a.n_vt * a.n_rbc));
    const dim3 blk(64 * kGradWaves);
    // Operand layouts: H and W stage-tiled or as stored; G_c stage-tiled, or K-blocked (the fp32
    // memory-lean backward, which reads H and W as stored).
    if (tiled_S > 0 && !g_tiled) return hipErrorInvalidValue;
    if (sh.act == Dt::BF16) {
        if (tiled_S > 0)
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<bf16_t, kGradWaves, kTiled, kTiled>), grid, blk, 0, s, a);
        else if (g_tiled)
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<bf16_t, kGradWaves, kRow, kTiled>), grid, blk, 0, s, a);
        else
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<bf16_t, kGradWaves, kRow, kKBlk>), grid, blk, 0, s, a);
    } else {
        if (tiled_S > 0)
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<float, kGradWaves, kTiled, kTiled>), grid, blk, 0, s, a);
        else if (g_tiled)
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<float, kGradWaves, kRow, kTiled>), grid, blk, 0, s, a);
        else
            KD_LAUNCH(kKindBwdGrad, s, (k_bwd_grad<float, kGradWaves, kRow, kKBlk>), grid, blk, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_grad_z(const Shape& sh, const float* zt, int64_t ldzt, int64_t zt_col0, const float* lse,
                         const float* pt, const float* grad_loss, int64_t c0, int64_t cc, const int32_t* plan_off,
                         const uint32_t* plan_ent, void* Gc, void* GT, int64_t ldgt, int64_t gt_col0,
                         hipStream_t s) {
    if (GT && (ldgt % 32 != 0 || gt_col0 % 32 != 0)) return hipErrorInvalidValue;
    GradArgs a;
    a.H = nullptr;
    a.W = nullptr;
    a.ldh = a.ldw = 0;
    a.zt = zt;
    a.ldzt = ldzt;
    a.zt_col0 = zt_col0;
    a.d = sh.d;
    a.V = sh.V;
    a.K = sh.K;
    a.c = kLog2e / sh.T;
    a.gsc = sh.T / sh.n_norm;
    a.grad = grad_loss;
    a.lse = lse;
    a.pt = pt;
    a.c0 = c0;
    a.cc = cc;
    a.off = plan_off;
    a.ent = plan_ent;
    a.n_vt = (int)((sh.V + kTileN - 1) / kTileN);
    a.n_rbc = (int)((cc + kTileM - 1) / kTileM);
    a.G = Gc;
    a.GT = GT;
    a.ldgt = ldgt;
    a.gt_col0 = gt_col0;
    a.ccp = round_up(cc, 32);
    const dim3 grid(grid_xcd((int64_t)a.n_vt * a.n_rbc));
    if (sh.act == Dt::BF16)
        KD_LAUNCH(kKindGradZ, s, k_grad_z<bf16_t>, grid, dim3(NTHR), 0, s, a);
    else
        KD_LAUNCH(kKindGradZ, s, k_grad_z<float>, grid, dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk(Dt dt, const void* X, int64_t ld, int64_t N, int64_t V, int64_t K, int32_t* idx, void* val,
                       hipStream_t s) {
    if (N > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t es = dt == Dt::BF16 ? 2 : 4, vec = 16 / es;
    // The register-resident pass takes rows that fill at least a third of its registers and
    // whose bases are 16-byte aligned, with K <= kTkrMaxK; the rows it cannot settle, and every
    // other problem, go through k_topk.
    const int64_t nvec = V / vec;
    const bool reg = K <= kTkrMaxK && nvec <= (int64_t)kTkrThreads * kTkrChunks &&
                     nvec * 3 >= (int64_t)kTkrThreads * kTkrChunks && ((uintptr_t)X % 16) == 0 &&
                     (ld * es) % 16 == 0;
    if (reg) {
        const unsigned grid = (unsigned)std::min<int64_t>(N, device_cus());
        if (dt == Dt::BF16)
            KD_LAUNCH(kKindTopk, s, k_topk_reg<bf16_t>, dim3(grid), dim3(kTkrThreads), 0, s, (const bf16_t*)X, ld, N,
                      (int)V, (int)K, idx, (bf16_t*)val);
        else
            KD_LAUNCH(kKindTopk, s, k_topk_reg<float>, dim3(grid), dim3(kTkrThreads), 0, s, (const float*)X, ld, N,
                      (int)V, (int)K, idx, (float*)val);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int flagged = reg ? 1 : 0;
    if (dt == Dt::BF16)
        KD_LAUNCH(kKindTopk, s, k_topk<bf16_t>, dim3((unsigned)N), dim3(NTHR), 0, s, (const bf16_t*)X, ld, N, (int)V,
                  (int)K, idx, (bf16_t*)val, flagged);
    else
        KD_LAUNCH(kKindTopk, s, k_topk<float>, dim3((unsigned)N), dim3(NTHR), 0, s, (const float*)X, ld, N, (int)V,
                  (int)K, idx, (float*)val, flagged);
    return hipGetLastError();
}

hipError_t launch_transpose(Dt dt, const void* src, int64_t lds, int64_t rows, int64_t cols, void* dst, int64_t kdst,
                            int64_t k0, int64_t rows_pad, hipStream_t s, void* tiled_copy) {
    const int64_t sw = dt == Dt::BF16 ? 32 : 16;
    if (kdst % sw != 0 || k0 % sw != 0 || k0 + rows_pad > kdst) return hipErrorInvalidValue;
    // the untransposed copy needs every row block of 256 covered: rows_pad a multiple of 256
    if (tiled_copy && rows_pad % kTileM != 0) return hipErrorInvalidValue;
    const int64_t S2 = tiled_stages(dt, cols);
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows_pad + 63) / 64));
    if (dt == Dt::BF16)
        KD_LAUNCH(kKindTranspose, s, k_transpose<bf16_t>, grid, dim3(NTHR), 0, s, (const bf16_t*)src, lds, rows, cols,
                  (bf16_t*)dst, kdst / sw, k0, rows_pad, (bf16_t*)tiled_copy, S2);
    else
        KD_LAUNCH(kKindTranspose, s, k_transpose<float>, grid, dim3(NTHR), 0, s, (const float*)src, lds, rows, cols,
                  (float*)dst, kdst / sw, k0, rows_pad, (float*)tiled_copy, S2);
    return hipGetLastError();
}

int64_t tiled_stages(Dt dt, int64_t cols) {
    const int64_t sw = dt == Dt::BF16 ? 32 : 16;
    return (cols + sw - 1) / sw;
}

int64_t tiled_bytes(Dt dt, int64_t rows, int64_t cols) {
    return round_up(rows, kTileM) * tiled_stages(dt, cols) * 64;
}

hipError_t launch_tile_rows(Dt dt, const void* src, int64_t ld, int64_t rows, int64_t cols, void* dst,
                            hipStream_t s) {
    const int64_t S = tiled_stages(dt, cols);
    const dim3 grid((unsigned)((S + 7) / 8), (unsigned)((rows + kTileM - 1) / kTileM));
    if (dt == Dt::BF16)
        KD_LAUNCH(kKindTranspose, s, k_tile_rows<bf16_t>, grid, dim3(NTHR), 0, s, (const bf16_t*)src, ld, rows, cols,
                  S, (bf16_t*)dst);
    else
        KD_LAUNCH(kKindTranspose, s, k_tile_rows<float>, grid, dim3(NTHR), 0, s, (const float*)src, ld, rows, cols, S,
                  (float*)dst);
    return hipGetLastError();
}

hipError_t launch_dh(const Shape& sh, const void* Gc, int64_t ldg, const void* W, const void* WT, int64_t c0,
                     int64_t cc, int n_split, float* part, void* dH, hipStream_t s, bool lean) {
    DhArgs a;
    a.G = Gc;
    a.ldg = ldg;
    a.Vp = round_up(sh.V, kTileN);
    a.W = WT ? WT : W;
    a.d = sh.d;
    a.V = sh.V;
    a.c0 = c0;
    a.cc = cc;
    a.n_split = n_split;
    a.kper = round_up((a.Vp + n_split - 1) / n_split, 64);
    a.part = part;
    a.dH = dH;
    // the wide tile: from W^T, or (the memory-lean backward, bf16) from W as stored
    const bool wide = WT || (lean && sh.act == Dt::BF16);
    a.n_nt = (int)((sh.d + (wide ? kWideN : kTileN) - 1) / (wide ? kWideN : kTileN));
    a.n_mt = (int)((cc + kTileM - 1) / kTileM);
    const dim3 grid(grid_xcd((int64_t)n_split * a.n_nt * a.n_mt));
    if (sh.act == Dt::BF16) {
        if (WT)
            KD_LAUNCH(kKindDh, s, (k_dh_w<bf16_t, kTiled>), grid, dim3(512), 0, s, a);
        else if (lean)  // bf16: G_c stage-tiled
            KD_LAUNCH(kKindDh, s, (k_dh_w<bf16_t, kTrans>), grid, dim3(512), 0, s, a);
        else
            KD_LAUNCH(kKindDh, s, (k_dh<bf16_t, false>), grid, dim3(NTHR), 0, s, a);
    } else {
        if (WT)
            KD_LAUNCH(kKindDh, s, (k_dh_w<float, kTiled>), grid, dim3(512), 0, s, a);
        else if (lean)  // fp32: G_c K-blocked
            KD_LAUNCH(kKindDh, s, (k_dh<float, true>), grid, dim3(NTHR), 0, s, a);
        else
            KD_LAUNCH(kKindDh, s, (k_dh<float, false>), grid, dim3(NTHR), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split <= 1) return e;
    const int64_t n4 = cc * sh.d / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((n4 + NTHR - 1) / NTHR, 4096);
    if (sh.act == Dt::BF16)
        KD_LAUNCH(kKindDhReduce, s, k_dh_reduce<bf16_t>, dim3(blocks), dim3(NTHR), 0, s, part, n_split, cc, sh.d, c0, dH);
    else
        KD_LAUNCH(kKindDhReduce, s, k_dh_reduce<float>, dim3(blocks), dim3(NTHR), 0, s, part, n_split, cc, sh.d, c0, dH);
    return hipGetLastError();
}

hipError_t launch_dw(const Shape& sh, const void* Gc, int64_t ldg, const void* H, int64_t c0, int64_t cc,
                     bool accumulate, float* dW, hipStream_t s, bool lean) {
    DwArgs a;
    a.G = Gc;
    a.ldg = ldg;
    a.g_blk = lean ? 1 : 0;  // the fp32 memory-lean G_c is K-blocked
    a.Vp = round_up(sh.V, kTileN);
    a.H = H;
    a.ldh = sh.d;
    a.d = sh.d;
    a.V = sh.V;
    a.c0 = c0;
    a.cc = cc;
    a.ccp = cc;
    a.accumulate = accumulate ? 1 : 0;
    a.dW = dW;
    a.n_mt = (int)(a.Vp / kTileM);
    if (lean && sh.act == Dt::BF16) {
        // the memory-lean backward: 256 x 320 tiles on the stage-tiled G_c and H as stored
        a.n_nt = (int)((sh.d + kWideN - 1) / kWideN);
        const dim3 grid(grid_xcd((int64_t)a.n_nt * a.n_mt));
        KD_LAUNCH(kKindDw, s, (k_dw_w<bf16_t, kTransT>), grid, dim3(512), 0, s, a);
        return hipGetLastError();
    }
    a.n_nt = (int)((sh.d + kTileN - 1) / kTileN);
    const dim3 grid(grid_xcd((int64_t)a.n_nt * a.n_mt));
    if (sh.act == Dt::BF16)
        KD_LAUNCH(kKindDw, s, k_dw<bf16_t>, grid, dim3(NTHR), 0, s, a);
    else
        KD_LAUNCH(kKindDw, s, k_dw<float>, grid, dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dw_t(const Shape& sh, const void* GT, int64_t ldgt, const void* HT, int64_t ldht, int64_t cc,
                       bool accumulate, float* dW, hipStream_t s) {
    DwArgs a;
    a.G = GT;
    a.ldg = ldgt;
    a.g_blk = 0;
    a.Vp = round_up(sh.V, kTileN);
    a.H = HT;
    a.ldh = ldht;
    a.d = sh.d;
    a.V = sh.V;
    a.c0 = 0;
    a.cc = cc;
    a.ccp = round_up(cc, 8);
    a.accumulate = accumulate ? 1 : 0;
    a.dW = dW;
    a.n_nt = (int)((sh.d + kWideN - 1) / kWideN);
    a.n_mt = (int)(a.Vp / kTileM);
    const dim3 grid(grid_xcd((int64_t)a.n_nt * a.n_mt));
    if (sh.act == Dt::BF16)
        KD_LAUNCH(kKindDw, s, (k_dw_w<bf16_t, kTiled>), grid, dim3(512), 0, s, a);
    else
        KD_LAUNCH(kKindDw, s, (k_dw_w<float, kTiled>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dense_logits(const Shape& sh, const void* H, const void* W, float* Z, int64_t ldz, hipStream_t s) {
    const dim3 grid(grid_xcd((ldz / kTileN) * ((sh.N + kTileM - 1) / kTileM)));
    if (sh.act == Dt::BF16)
        KD_LAUNCH(kKindDenseLogits, s, k_dense_logits<bf16_t>, grid, dim3(NTHR), 0, s, H, W, sh.N, sh.d, sh.V, Z, ldz);
    else
        KD_LAUNCH(kKindDenseLogits, s, k_dense_logits<float>, grid, dim3(NTHR), 0, s, H, W, sh.N, sh.d, sh.V, Z, ldz);
    return hipGetLastError();
}

hipError_t launch_dense_rows(const Shape& sh, float* Z, float* P, int64_t ldz, const int32_t* idx, const void* tlog,
                             const float* grad_loss, float* lse, float* row_kl, double* row_sum, void* G,
                             int64_t ldg, hipStream_t s) {
    (void)G;
    (void)ldg;
    KD_LAUNCH(kKindDenseRows, s, k_dense_rows, dim3((unsigned)sh.N), dim3(NTHR), 0, s, Z, P, ldz, sh.V, (int)sh.K, sh.T,
                       sh.T / sh.n_norm, idx, tlog, sh.tlog, grad_loss, lse, row_kl, row_sum,
                       sh.act == Dt::BF16 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_sum_rows(const Shape& sh, const double* row_sum, double* blk_sum, int* n_blk, hipStream_t s) {
    const int nb = (int)((sh.N + 1023) / 1024);
    KD_LAUNCH(kKindSumRows, s, k_sum_rows, dim3(nb), dim3(NTHR), 0, s, row_sum, sh.N, blk_sum);
    if (n_blk) *n_blk = nb;
    return hipGetLastError();
}

}  // namespace kdkl
