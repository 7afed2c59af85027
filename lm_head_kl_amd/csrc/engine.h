// MFMA tile engine for gfx950, shared by every GEMM-shaped kernel of libkdkl.
//
// A workgroup computes one fp32 tile of C = A B^T over a K range, with the accumulators in
// registers. Four variants:
//   gemm_tile       256 x 256, four waves (2 x 2, 128 x 128 each as 4 x 4 blocks of
//                   v_mfma_f32_32x32x16_bf16 / 32x32x2_f32, accumulators in AGPRs), two LDS
//                   stages of a full K step; takes M/N-contiguous operands (dense path, fp32
//                   memory-lean backward).
//   gemm_tile_kk    same tile on K-contiguous operands, four LDS stages of half a K step,
//                   four or eight waves (dense logits).
//   gemm_tile_kk16  same tile and stages, eight waves (2 x 4, 128 x 64 each as 8 x 4 blocks of
//                   v_mfma_f32_16x16x32_bf16 / 16x16x4_f32): forward and gradient kernels.
//   gemm_tile_w16   256 x 320, eight waves (2 x 4, 128 x 80 each as 8 x 5 16x16 blocks): dH, dW;
//                   either operand may also be M/N contiguous (kTrans, kTransT), reaching the
//                   MFMAs through LDS transpose reads (bf16 memory-lean backward).
//
// Operands reach LDS in 16-byte chunks:
//   - K contiguous (element (mn, k) at src[mn*ld + k]): buffer_load_dwordx4 with the LDS
//     destination bit, straight from memory into LDS. No VGPRs and no ds_write are used.
//     A wave instruction fills 64 consecutive LDS chunks, so each lane fetches the global
//     chunk that belongs at its destination under the stage's swizzle.
//   - M/N contiguous (element (mn, k) at src[k*ld + mn]) in gemm_tile: buffer loads of
//     8 x 8 (bf16) or 4 x 4 (fp32) blocks into VGPRs, transposed in registers and written with
//     ds_write_b128;
//   - M/N contiguous in gemm_tile_w16 (bf16): the same LDS DMA as K-contiguous operands, rows of
//     k into LDS as they lie, and ds_read_b64_tr_b16 pairs transpose them into fragments.
// Rows and k beyond the operand's limits are read through an out-of-range offset of the
// buffer descriptor. The hardware returns zeros for those, so the loop has no branches.
//
// gemm_tile's LDS layout: [256 rows][8 chunks of 16 bytes]. Chunk c of row r sits at
// c ^ ((r ^ (r >> 3)) & 7). This is conflict free for the MFMA fragment reads (32 rows, one
// chunk column), for the DMA fill (8 rows x 8 chunks per 1 KB), and for the transposed
// writes (rows 8 apart). The half-K stages use [rows][4 chunks] with their own swizzle (swz4).
//
// MFMA lane layouts (checked on gfx950 hardware):
//   32x32x16 bf16: lane l supplies A[m = l%32][k = 8*(l/32) + 0..7], and B likewise with n.
//   32x32x2 f32:   lane l supplies A[m = l%32][k = l/32].
//   Accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
//   16x16x32 bf16: lane l supplies A[m = l%16][k = 8*(l/16) + 0..7]; accumulator element v of
//                  lane l: row 4*(l/16) + v, column l%16.
// The DMA fill places lane l's 16 bytes at M0 + 16*l; an out-of-range offset writes zeros
// (also checked on hardware).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kdkl_internal.h"

namespace kdkl {

typedef uint16_t bf16_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NTHR = 256;
constexpr int NCH = 8;                       // 16-byte chunks per tile row per K step
constexpr int TILE_CHUNKS = kTileM * NCH;    // 2048 chunks = 32 KB per operand per stage
// A kernel's operand stages sit at LDS offset 0, in its only LDS array (anything else it keeps in
// LDS goes after them in the same array): with a second LDS object that the compiler placed in
// front of the stages, the gradient kernel's mainloop ran 50% slower.
constexpr int LDS_CHUNKS = 4 * TILE_CHUNKS;  // 2 stages x 2 operands = 128 KB
constexpr uint32_t kOOB = 0x7FFFFFF0u;       // descriptor range; offsets >= it read as zero

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int VEC = 8; static constexpr int BK = 64; };
template <> struct Elem<float> { static constexpr int VEC = 4; static constexpr int BK = 32; };

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// The base is the same in every lane; say so, so that the descriptor lives in SGPRs and the
// loads need no waterfall loop.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(base)), (short)0, (int)kOOB,
                                             0x00020000);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Position of a thread in the workgroup's wave grid over the 256 x 256 tile. NW = 4 waves
// form a 2 x 2 grid (128 x 128 per wave, 4 x 4 MFMA blocks); NW = 8 waves a 2 x 4 grid
// (128 x 64 per wave, 4 x 2 blocks, two waves per SIMD).
template <int NW>
struct WaveIdN {
    static constexpr int JN = 16 / NW;       // MFMA blocks per wave along N
    static constexpr int NSPAN = 32 * JN;    // tile columns per wave
    int tid, lane, w, wm, wn, h, lr;
    __device__ WaveIdN() {
        tid = threadIdx.x;
        lane = tid & 63;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        wm = w / (NW / 2);
        wn = w % (NW / 2);
        h = lane >> 5;
        lr = lane & 31;
    }
    // A copy whose per-lane fields the compiler must recompute where it is taken. Epilogues
    // inside persistent tile loops take one, so their many LDS addresses are not hoisted out
    // of the loop and kept live (spilled) across the mainloop.
    __device__ __forceinline__ WaveIdN fresh() const {
        WaveIdN c = *this;
        asm volatile("v_mov_b32 %0, %1" : "=v"(c.tid) : "v"(tid));
        c.lane = c.tid & 63;
        c.h = c.lane >> 5;
        c.lr = c.lane & 31;
        return c;
    }
};
using WaveId = WaveIdN<4>;

template <typename T> __device__ __forceinline__ void mma(f32x16& c, const u32x4& a, const u32x4& b);
template <> __device__ __forceinline__ void mma<bf16_t>(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                c, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma<float>(f32x16& c, const u32x4& a, const u32x4& b) {
    // A 16-byte chunk holds 4 consecutive k and the two lane halves hold neighbouring chunks.
    // Instruction i takes element i of each, so the four together cover 8 distinct k, the
    // same ones for A and B.
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
}

// ------------------------------------------------------------------------------------------
// K-contiguous operand, filled by DMA. Wave w's instruction t fills LDS chunks
// 256t + 64w + lane, i.e. row 32t + 8w + lane/8, physical chunk lane%8.
// BLK selects the K-blocked layout (K cut into blocks of 256, each a row-major [R][256] slab;
// ld is then the row count R). A K step (64 bf16 / 32 fp32) never straddles a block.
template <typename T, bool BLK = false>
struct KOperand {
    static constexpr int VEC = Elem<T>::VEC;
    const char* base;  // &src[mn0*ld] (row-major) or &src[mn0*256] in block 0 (uniform)
    int64_t blk_bytes; // K-blocked: bytes per block
    uint32_t off[8];   // byte offset of this lane's chunk for instruction t at k = 0, or kOOB
    int chunk[2];      // logical chunk (k/VEC within the step) for even / odd t

    __device__ __forceinline__ void init(const T* src, int64_t ld, int64_t mn0, int64_t mn_lim, const WaveId& id) {
        const int64_t row_ld = BLK ? 256 : ld;
        base = (const char*)(src + mn0 * row_ld);
        blk_bytes = BLK ? ld * 256 * (int64_t)sizeof(T) : 0;
        const int r8 = id.lane >> 3, p = id.lane & 7;
#pragma unroll
        for (int t = 0; t < 2; ++t) chunk[t] = p ^ ((r8 ^ (4 * t + id.w)) & 7);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 32 * t + 8 * id.w + r8;
            off[t] = mn0 + row < mn_lim ? (uint32_t)((row * row_ld + chunk[t & 1] * VEC) * (int64_t)sizeof(T)) : kOOB;
        }
    }
    // Enqueue the K step starting at k0 into the LDS tile (no wait).
    __device__ __forceinline__ void issue(u32x4* tile, int64_t k0, int64_t k_lim, const WaveId& id) const {
        const char* b = BLK ? base + (k0 >> 8) * blk_bytes + (k0 & 255) * (int64_t)sizeof(T)
                            : base + k0 * (int64_t)sizeof(T);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(b);
        const int64_t kc = (k_lim - k0 + VEC - 1) / VEC;  // chunks of this step inside the K range
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t o = chunk[t & 1] < kc ? off[t] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + 256 * t + 64 * id.w), 16, (int)o, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void commit(u32x4*, const WaveId&) const {}
};

// M/N-contiguous operand, through VGPRs with an in-register transpose.
template <typename T> struct MNOperand;

template <>
struct MNOperand<bf16_t> {
    // thread: mnb = tid%32 (8 mn), kb = tid/32 (8 k); loads 8 rows of 16 bytes.
    const char* base;  // &src[mn0] (uniform)
    int64_t ldb;       // row stride in bytes
    uint32_t off0;     // (kb*8)*ldb + mnb*16, or kOOB if the mn block is outside
    int kb;
    u32x4 r[8];

    __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int64_t mn0, int64_t mn_lim,
                                         const WaveId& id) {
        base = (const char*)(src + mn0);
        ldb = ld * 2;
        const int mnb = id.tid & 31;
        kb = id.tid >> 5;
        off0 = mn0 + mnb * 8 < mn_lim ? (uint32_t)(kb * 8 * ldb + mnb * 16) : kOOB;
    }
    __device__ __forceinline__ void issue(u32x4*, int64_t k0, int64_t k_lim, const WaveId&) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ldb);
        const int64_t kr = k_lim - k0 - kb * 8;  // rows of this thread's block inside the K range
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint32_t o = (kk < kr && off0 != kOOB) ? off0 + (uint32_t)(kk * ldb) : kOOB;
            r[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0));
        }
    }
    __device__ __forceinline__ void commit(u32x4* tile, const WaveId& id) const {
        const int mnb = id.tid & 31;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // row i of the transposed block: element i of each of the 8 loaded k-rows
            const int wsel = i >> 1, sh = 16 * (i & 1);
            u32x4 y;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = (r[2 * p][wsel] >> sh) & 0xffffu;
                const uint32_t hi = (r[2 * p + 1][wsel] >> sh) & 0xffffu;
                y[p] = lo | (hi << 16);
            }
            const int row = mnb * 8 + i;
            tile[row * NCH + swz(row, kb)] = y;
        }
    }
};

template <>
struct MNOperand<float> {
    // two 4(k) x 4(mn) blocks per thread: q = tid + 256*t, mnb = q%64, kb = q/64.
    const char* base;
    int64_t ldb;
    uint32_t off0[2];
    u32x4 r[8];

    __device__ __forceinline__ void init(const float* src, int64_t ld, int64_t mn0, int64_t mn_lim,
                                         const WaveId& id) {
        base = (const char*)(src + mn0);
        ldb = ld * 4;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int q = id.tid + NTHR * t, mnb = q & 63, kb = q >> 6;
            off0[t] = mn0 + mnb * 4 < mn_lim ? (uint32_t)(kb * 4 * ldb + mnb * 16) : kOOB;
        }
    }
    __device__ __forceinline__ void issue(u32x4*, int64_t k0, int64_t k_lim, const WaveId& id) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ldb);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kb = (id.tid + NTHR * t) >> 6;
            const int64_t kr = k_lim - k0 - kb * 4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t o = (kk < kr && off0[t] != kOOB) ? off0[t] + (uint32_t)(kk * ldb) : kOOB;
                r[t * 4 + kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0));
            }
        }
    }
    __device__ __forceinline__ void commit(u32x4* tile, const WaveId& id) const {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int q = id.tid + NTHR * t, mnb = q & 63, kb = q >> 6;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 y{r[t * 4 + 0][i], r[t * 4 + 1][i], r[t * 4 + 2][i], r[t * 4 + 3][i]};
                const int row = mnb * 4 + i;
                tile[row * NCH + swz(row, kb)] = y;
            }
        }
    }
};

template <typename T, bool KMAJ, bool BLK = false> struct OperandSel { using type = KOperand<T, BLK>; };
template <typename T, bool BLK> struct OperandSel<T, false, BLK> { using type = MNOperand<T>; };

// One K step from LDS: for each of the 4 k-groups, 4 A and 4 B fragments and 16 MFMAs.
// Fragments are double-buffered so the reads of group g+1 overlap the MFMAs of group g.
template <typename T>
__device__ __forceinline__ void compute_stage(f32x16 (&acc)[4][4], const u32x4* tA, const u32x4* tB,
                                              const WaveId& id) {
    u32x4 fa[2][4], fb[2][4];
    auto read = [&](int g, u32x4(&a)[4], u32x4(&b)[4]) {
        const int c = 2 * g + id.h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = id.wm * 128 + i * 32 + id.lr;
            a[i] = tA[row * NCH + swz(row, c)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = id.wn * 128 + j * 32 + id.lr;
            b[j] = tB[row * NCH + swz(row, c)];
        }
    };
    read(0, fa[0], fb[0]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (g < 3) read(g + 1, fa[(g + 1) & 1], fb[(g + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma<T>(acc[i][j], fa[g & 1][i], fb[g & 1][j]);
    }
}

// acc = A[m0:m0+256, k_begin:k_end] B[n0:n0+256, k_begin:k_end]^T.
// AK / BK: operand is K contiguous. ka_lim / kb_lim: first k each operand may not read
// (multiples of the 16-byte vector width). Rows at or past m_lim / n_lim read as zero.
// BLKA: A is K contiguous in the K-blocked layout (lda = its row count).
// Ends with a barrier, so the LDS may be reused right away.
template <typename T, bool AK, bool BKM, bool BLKA = false>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], u32x4* L, const WaveId& id,
                                          const T* A, int64_t lda, int64_t m0, int64_t m_lim, int64_t ka_lim,
                                          const T* B, int64_t ldb, int64_t n0, int64_t n_lim, int64_t kb_lim,
                                          int64_t k_begin, int64_t k_end) {
    constexpr int BK = Elem<T>::BK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const int nk = (int)((k_end - k_begin + BK - 1) / BK);
    if (nk <= 0) return;
    static_assert(AK || !BLKA, "the K-blocked layout is for K-contiguous operands");
    typename OperandSel<T, AK, BLKA>::type opA;
    typename OperandSel<T, BKM>::type opB;
    opA.init(A, lda, m0, m_lim, id);
    opB.init(B, ldb, n0, n_lim, id);
    opA.issue(L, k_begin, ka_lim, id);
    opB.issue(L + TILE_CHUNKS, k_begin, kb_lim, id);
    wait_vmem();
    opA.commit(L, id);
    opB.commit(L + TILE_CHUNKS, id);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        u32x4* nA = L + (2 * (cur ^ 1)) * TILE_CHUNKS;
        u32x4* nB = nA + TILE_CHUNKS;
        if (more) {
            const int64_t k0 = k_begin + (int64_t)(kt + 1) * BK;
            opA.issue(nA, k0, ka_lim, id);
            opB.issue(nB, k0, kb_lim, id);
        }
        compute_stage<T>(acc, L + (2 * cur) * TILE_CHUNKS, L + (2 * cur + 1) * TILE_CHUNKS, id);
        if (more) {
            wait_vmem();
            opA.commit(nA, id);
            opB.commit(nB, id);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// Deep-pipelined variant for two K-contiguous operands: four LDS stages of half the K step
// (32 bf16 / 16 fp32), each tile [256 rows][4 chunks]. DMA loads run three stages ahead of
// the MFMAs, which covers memory latency beyond one step. The chunk swizzle for 4-chunk rows
// is c ^ (((r >> 2) ^ (r >> 1)) & 3). It is conflict free for fragment reads served 8 or 16
// lanes at a time.
constexpr int NCH4 = 4;
constexpr int TILE4 = kTileM * NCH4;  // 1024 chunks = 16 KB per operand per stage
__device__ __forceinline__ int swz4(int r, int c) { return c ^ (((r >> 2) ^ (r >> 1)) & 3); }

// Three operand layouts (LAY):
//   kRow    row-major: element (mn, k) at src[mn*ld + k];
//   kKBlk   K-blocked: the K axis cut into blocks of 256, each block a row-major [R][256] slab:
//           element (mn, k) at src[((k >> 8)*R + mn)*256 + (k & 255)], with ld = R;
//   kTiled  stage-tiled: rows cut into blocks of RB (the tile's rows) and K into stages of SW =
//           64 bytes, each (row block, stage) a contiguous [RB][SW] block:
//           element (mn, k) at src[((mn / RB)*S + k / SW)*RB*SW + (mn % RB)*SW + k % SW], with
//           ld = S, the stages per row block; K is zero-padded to S*SW and rows to whole blocks.
// One stage of a tile is 64 bytes of each of its rows. Row-major and K-blocked operands give it
// as 64-byte pieces of separate 128-byte lines, the second half of each line following one stage
// later; a stage-tiled operand gives it as one contiguous block, every line whole. At the
// gpt-oss head the same mainloop runs 15-18 % faster on stage-tiled operands.
//   kTrans  M/N-contiguous (bf16, wide tile only): each source row holds one K index, and the
//           tile's M or N entries are contiguous in it: element (mn, k) at src[k*ld + mn - mn0]
//           for a src that the caller points at the tile's first column. Read through LDS
//           transpose reads (see KOperandTR).
//   kTransT the same, stage-tiled with the roles of rows and columns exchanged: K runs along
//           the rows (blocks of 256), M/N along the 64-byte stages: element (mn, k) at
//           src[((k/256)*ld + (mn-mn0)/32)*8192 + (k%256)*32 + (mn-mn0)%32], src at the tile's
//           first column, ld the stages per row block. Each stage's 32 K rows of a 32-column
//           block are then one contiguous 2 KB piece.
enum Lay : int { kRow = 0, kKBlk = 1, kTiled = 2, kTrans = 3, kTransT = 4 };

template <typename T, int LAY = kRow, int NW = 4>
struct KOperand4 {
    static constexpr int TPI = 16 / NW;  // DMA instructions per wave per stage
    static constexpr int VEC = Elem<T>::VEC;
    static constexpr bool BLK = LAY == kKBlk;
    // row-major: tile origin &src[mn0*ld], k0 in the scalar offset; stage-tiled: the tile's
    // first block, the stage's block in the scalar offset
    __amdgpu_buffer_rsrc_t rsrc;
    const char* base;             // K-blocked: &src[mn0*256] in block 0
    int64_t blk_bytes;            // K-blocked: bytes per block
    uint32_t off[TPI];
    int chunk;
    // Wave w's instruction t fills chunks 64 NW t + 64w + lane: row 16 NW t + 16w + lane/4, slot lane%4.
    // A stage-tiled operand needs mn0 % kTileM == 0.
    __device__ __forceinline__ void init(const T* src, int64_t ld, int64_t mn0, int64_t mn_lim,
                                         const WaveIdN<NW>& id) {
        const int64_t row_ld = BLK ? 256 : LAY == kTiled ? 4 * VEC : ld;
        if constexpr (BLK) {
            base = (const char*)uniform_ptr(src + mn0 * 256);
            blk_bytes = ld * 256 * (int64_t)sizeof(T);
        } else if constexpr (LAY == kTiled) {
            rsrc = make_rsrc(src + (mn0 / kTileM) * ld * (kTileM * 4 * VEC));
        } else {
            rsrc = make_rsrc(src + mn0 * ld);
        }
        chunk = (id.lane & 3) ^ (((id.lane >> 4) ^ (id.lane >> 3)) & 3);
#pragma unroll
        for (int t = 0; t < TPI; ++t) {
            const int row = 16 * NW * t + 16 * id.w + (id.lane >> 2);
            off[t] = mn0 + row < mn_lim ? (uint32_t)((row * row_ld + chunk * VEC) * (int64_t)sizeof(T)) : kOOB;
        }
    }
    // Load instruction t of the K step at k0 into the stage tile. Chunks at or past k_lim, and
    // every chunk when `live` is false, read as zero (no memory access). `full` (uniform) says
    // the whole step is inside the K range. A step never straddles a K block (k0 is a multiple
    // of the step and the step divides 256).
    __device__ __forceinline__ void issue_one(u32x4* tile, int t, int64_t k0, int64_t k_lim, bool full, bool live,
                                              const WaveIdN<NW>& id) const {
        const bool in = live && (full || (int64_t)chunk * VEC < k_lim - k0);
        if constexpr (BLK) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (k0 >> 8) * blk_bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + 64 * NW * t + 64 * id.w), 16,
                                                     (int)(in ? off[t] : kOOB), (int)((k0 & 255) * (int64_t)sizeof(T)),
                                                     0, 0);
        } else if constexpr (LAY == kTiled) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + 64 * NW * t + 64 * id.w), 16,
                                                     (int)(in ? off[t] : kOOB),
                                                     (int)((k0 / (4 * VEC)) * (kTileM * 64)), 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + 64 * NW * t + 64 * id.w), 16,
                                                     (int)(in ? off[t] : kOOB), (int)(k0 * (int64_t)sizeof(T)), 0, 0);
        }
    }
    __device__ __forceinline__ void issue(u32x4* tile, int64_t k0, int64_t k_lim, bool live,
                                          const WaveIdN<NW>& id) const {
        const bool full = k0 + Elem<T>::BK / 2 <= k_lim;
#pragma unroll
        for (int t = 0; t < TPI; ++t) issue_one(tile, t, k0, k_lim, full, live, id);
    }
};

// Fragments of one k-group (g = 0, 1) of a 4-chunk stage: 4 A and 4 B chunks.
template <typename T, int NW>
__device__ __forceinline__ void read_frags4(u32x4 (&fa)[4], u32x4 (&fb)[16 / NW], const u32x4* tA, const u32x4* tB,
                                            int g, const WaveIdN<NW>& id) {
    const int c = 2 * g + id.h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = id.wm * 128 + i * 32 + id.lr;
        fa[i] = tA[row * NCH4 + swz4(row, c)];
    }
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
        const int row = id.wn * (512 / NW) + j * 32 + id.lr;
        fb[j] = tB[row * NCH4 + swz4(row, c)];
    }
}

template <typename T, int JN>
__device__ __forceinline__ void mma_block(f32x16 (&acc)[4][JN], const u32x4 (&fa)[4], const u32x4 (&fb)[JN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) mma<T>(acc[i][j], fa[i], fb[j]);
}

template <int N> __device__ __forceinline__ void wait_vmem_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Barrier for an LDS hand-off only. __syncthreads() also fences global memory at workgroup
// scope, so after global stores (a previous tile's epilogue) it waits for all of them and for
// every DMA load still in flight; this waits for the wave's LDS operations alone. DMA writes
// into LDS are covered by the caller's vmcnt wait.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

#define KD_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
// sched_group_barrier masks
#define KD_SG_MFMA 0x008
#define KD_SG_VMEM_RD 0x020
#define KD_SG_DS_RD 0x100

// Same contract as gemm_tile with both operands K contiguous.
// Four LDS stages of half a K step. Schedule of stage kt (k-groups g0, g1; fragment sets F0, F1):
//   [MFMA(F0) interleaved with reads F1 <- (kt, g1)]
//   wait for stage kt+1, barrier
//   [MFMA(F1) interleaved with DMA of stage kt+4 into stage kt's buffer and reads F0 <- (kt+1, g0)]
// Stage kt's buffer is free after that barrier (its last fragments were read before it), so
// the DMA runs four stages ahead. Every LDS read is issued one MFMA block ahead of its use.
// BA / BB select the layout of A / B (Lay; lda / ldb is then the row stride, the row count or
// the stages per row block).
// NW is the wave count of the workgroup (4 or 8, see WaveIdN); acc is [4][16/NW].
template <typename T, int BA = kRow, int BB = kRow, int NW = 4>
__device__ __forceinline__ void gemm_tile_kk(f32x16 (&acc)[4][16 / NW], u32x4* L, const WaveIdN<NW>& id,
                                             const T* A, int64_t lda, int64_t m0, int64_t m_lim, int64_t ka_lim,
                                             const T* B, int64_t ldb, int64_t n0, int64_t n_lim, int64_t kb_lim,
                                             int64_t k_begin, int64_t k_end) {
    constexpr int BKH = Elem<T>::BK / 2;
    constexpr int JN = 16 / NW;   // B fragments (and MFMA columns) per wave
    constexpr int TPI = 16 / NW;  // DMA instructions per operand per wave per stage
    constexpr int NFR = 4 + JN;   // fragment reads per k-group
    constexpr int NMM = 4 * JN;   // MFMAs per k-group
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) acc[i][j] = f32x16{};
    const int nk = (int)((k_end - k_begin + BKH - 1) / BKH);
    if (nk <= 0) return;
    KOperand4<T, BA, NW> opA;
    KOperand4<T, BB, NW> opB;
    opA.init(A, lda, m0, m_lim, id);
    opB.init(B, ldb, n0, n_lim, id);
    auto stageA = [&](int s) { return L + (2 * (s & 3)) * TILE4; };
    auto stageB = [&](int s) { return L + (2 * (s & 3) + 1) * TILE4; };
    auto kof = [&](int s) { return k_begin + (int64_t)s * BKH; };
    // Every stage slot issues its 2 TPI loads, live or not, so the wait counts are constant:
    // stage s is complete once at most the 3 (prologue) or 2 (loop) later stages are in flight.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        opA.issue(stageA(s), kof(s), ka_lim, s < nk, id);
        opB.issue(stageB(s), kof(s), kb_lim, s < nk, id);
    }
    wait_vmem_le<6 * TPI>();
    lds_barrier();
    u32x4 f0a[4], f0b[JN], f1a[4], f1b[JN];
    read_frags4<T, NW>(f0a, f0b, stageA(0), stageB(0), 0, id);
    for (int kt = 0; kt + 1 < nk; ++kt) {
        KD_SCHED_FENCE();
        read_frags4<T, NW>(f1a, f1b, stageA(kt), stageB(kt), 1, id);
        mma_block<T, JN>(acc, f0a, f0b);
#pragma unroll
        for (int q = 0; q < NFR; ++q) {
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, NMM - NFR, 0);
        KD_SCHED_FENCE();
        wait_vmem_le<4 * TPI>();  // stage kt+1 complete; kt+2 and kt+3 may be in flight
        lds_barrier();
        KD_SCHED_FENCE();
        {
            const int s = kt + 4;
            const bool live = s < nk;
            const bool fa = kof(s) + BKH <= ka_lim, fb = kof(s) + BKH <= kb_lim;
#pragma unroll
            for (int t = 0; t < TPI; ++t) {
                opA.issue_one(stageA(s), t, kof(s), ka_lim, fa, live, id);
                opB.issue_one(stageB(s), t, kof(s), kb_lim, fb, live, id);
            }
        }
        read_frags4<T, NW>(f0a, f0b, stageA(kt + 1), stageB(kt + 1), 0, id);
        mma_block<T, JN>(acc, f1a, f1b);
        if constexpr (NW == 4) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_VMEM_RD, 1, 1);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, 1, 1);
            }
        } else {
            // 8 MFMAs carry 4 DMA issues and 6 fragment reads
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_VMEM_RD, 1, 1);
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
        }
        KD_SCHED_FENCE();
    }
    // last stage
    KD_SCHED_FENCE();
    read_frags4<T, NW>(f1a, f1b, stageA(nk - 1), stageB(nk - 1), 1, id);
    KD_SCHED_FENCE();
    mma_block<T, JN>(acc, f0a, f0b);
    KD_SCHED_FENCE();
    mma_block<T, JN>(acc, f1a, f1b);
    KD_SCHED_FENCE();
    wait_vmem_le<0>();  // no zero-fill may land after the caller reuses the LDS
    __syncthreads();
}

// ------------------------------------------------------------------------------------------
// 16 x 16 blocks for the 256 x 256 tile. v_mfma_f32_16x16x32_bf16 does half the work of a
// 32x32x16 in half the cycles but draws less power per FLOP, so at the chip's power limit a
// mainloop on it runs about 7% faster. Layout of a 16 x 16 fp32 block (f32x4): lane l holds
// column l % 16 and rows 4 (l / 16) + 0..3. A fragment is one 16-byte chunk per lane: row
// l % 16 of the block and chunk l / 16 of the stage's four (K32 bf16 or K16 fp32), so a stage
// is one k-group. The fp32 path issues four v_mfma_f32_16x16x4_f32, instruction i taking
// element i of every lane's chunk; lane group g then supplies k = 4g + i, the same k in A and B.
template <typename T> __device__ __forceinline__ void mma16(f32x4& c, const u32x4& a, const u32x4& b);
template <> __device__ __forceinline__ void mma16<bf16_t>(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                0, 0);
}
template <> __device__ __forceinline__ void mma16<float>(f32x4& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
}
template <typename T> struct Mfma16Count { static constexpr int N = sizeof(T) == 2 ? 1 : 4; };

// Fragment of the 16-row block whose first row is r0 (in a stage's A or B region).
__device__ __forceinline__ u32x4 frag16(const u32x4* S, int r0, int lane) {
    const int row = r0 + (lane & 15);
    return S[row * NCH4 + swz4(row, lane >> 4)];
}

// Same contract as gemm_tile_kk on eight waves, 16 x 16 blocks: each wave holds 128 x 64 as
// 8 x 4 blocks, acc[i][j] at tile rows wm*128 + 16i, columns wn*64 + 16j. Stage k splits by A
// rows: part 0 = rows 0-3 (A rows 4-7 of the stage read meanwhile), barrier, part 1 = rows 4-7
// (the DMA of stage k+4 issued, A rows 0-3 and B of stage k+1 read meanwhile). B alternates
// between two register sets, so the loop runs two stages per trip.
template <typename T, int BA = kRow, int BB = kRow>
__device__ __forceinline__ void gemm_tile_kk16(f32x4 (&acc)[8][4], u32x4* L, const WaveIdN<8>& id, const T* A,
                                               int64_t lda, int64_t m0, int64_t m_lim, int64_t ka_lim, const T* B,
                                               int64_t ldb, int64_t n0, int64_t n_lim, int64_t kb_lim,
                                               int64_t k_begin, int64_t k_end) {
    constexpr int BKH = Elem<T>::BK / 2;
    constexpr int TPI = 2;  // DMA instructions per operand per wave per stage
    constexpr int MM = Mfma16Count<T>::N;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = (int)((k_end - k_begin + BKH - 1) / BKH);
    if (nk <= 0) return;
    KOperand4<T, BA, 8> opA;
    KOperand4<T, BB, 8> opB;
    opA.init(A, lda, m0, m_lim, id);
    opB.init(B, ldb, n0, n_lim, id);
    auto stageA = [&](int s) { return L + (2 * (s & 3)) * TILE4; };
    auto stageB = [&](int s) { return L + (2 * (s & 3) + 1) * TILE4; };
    auto kof = [&](int s) { return k_begin + (int64_t)s * BKH; };
    u32x4 fa[8], fb[2][4];
    auto rdA = [&](int i0, int s) {
#pragma unroll
        for (int i = i0; i < i0 + 4; ++i) fa[i] = frag16(stageA(s), id.wm * 128 + 16 * i, id.lane);
    };
    auto rdB = [&](u32x4 (&b)[4], int s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = frag16(stageB(s), id.wn * 64 + 16 * j, id.lane);
    };
    auto stage = [&](int k, const u32x4 (&bc)[4], u32x4 (&bn)[4], bool more) {
        KD_SCHED_FENCE();
        rdA(4, k);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma16<T>(acc[i][j], fa[i], bc[j]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 3 * MM, 0);
            __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 4 * MM, 0);
        KD_SCHED_FENCE();
        if (more)
            wait_vmem_le<4 * TPI>();  // stage k+1 complete; k+2 and k+3 may be in flight
        else
            wait_vmem_le<0>();
        lds_barrier();
        KD_SCHED_FENCE();
        if (more) {
            const int s = k + 4;
            const bool live = s < nk;
            const bool fa_ = kof(s) + BKH <= ka_lim, fb_ = kof(s) + BKH <= kb_lim;
#pragma unroll
            for (int t = 0; t < TPI; ++t) {
                opA.issue_one(stageA(s), t, kof(s), ka_lim, fa_, live, id);
                opB.issue_one(stageB(s), t, kof(s), kb_lim, fb_, live, id);
            }
            rdA(0, k + 1);
            rdB(bn, k + 1);
        }
#pragma unroll
        for (int i = 4; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma16<T>(acc[i][j], fa[i], bc[j]);
        if (more) {
            // 16 MFMAs carry 4 DMA issues and 8 fragment reads
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, MM, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_VMEM_RD, 1, 1);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, MM, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, 1, 1);
            }
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 4 * MM, 1);
        }
        KD_SCHED_FENCE();
    };
    // Every stage slot issues its 2 TPI loads, live or not, so the wait counts are constant.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        opA.issue(stageA(s), kof(s), ka_lim, s < nk, id);
        opB.issue(stageB(s), kof(s), kb_lim, s < nk, id);
    }
    wait_vmem_le<6 * TPI>();
    lds_barrier();
    rdA(0, 0);
    rdB(fb[0], 0);
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
        stage(kt, fb[0], fb[1], true);
        stage(kt + 1, fb[1], fb[0], true);
    }
    // the last one or two stages
    stage(kt, fb[0], fb[1], kt + 1 < nk);
    if (kt + 1 < nk) stage(kt + 1, fb[1], fb[0], false);
    wait_vmem_le<0>();  // no zero-fill may land after the caller reuses the LDS
    __syncthreads();
}

// ------------------------------------------------------------------------------------------
// Wide tile: 256 x 320 (M x N), for products whose N is the hidden size d. d = 2880 is 9 x 320
// but 11.25 x 256, so 256-wide column tiles waste a quarter of their last tile; a 320-wide tile
// also moves about 10 % fewer operand bytes per FLOP. The stage layout, swizzle and pipeline are
// those of gemm_tile_kk: four stages of half a K step, A [256][4 chunks] + B [320][4 chunks]
// = 36 KB each. B takes 20 DMA instructions per stage: waves 0-3 issue three, waves 4-7 two and
// a third with an out-of-range offset (no memory access) into a 1 KB dummy slot of their own,
// so every wave issues five and the wait counts stay constant.
constexpr int kWideN = 320;
constexpr int WST = (kTileM + kWideN) * NCH4;           // chunks per stage (A then B)
constexpr int WIDE_LDS_CHUNKS = 4 * WST + 4 * 64;        // four stages + four dummy slots = 148 KB

// Operand of NI 16-row groups per wave (A: NI = 2 covers 256 rows; B: NI = 3 covers 320 rows,
// the third group of waves 4-7 being the dummy). Layouts as KOperand4; a stage-tiled operand has
// row blocks of the tile's rows (256 or 320) and needs mn0 to be a multiple of them.
template <typename T, int LAY, int NI, int ROWS>
struct KOperandW {
    static constexpr int VEC = Elem<T>::VEC;
    static constexpr bool BLK = LAY == kKBlk;
    __amdgpu_buffer_rsrc_t rsrc;
    const char* base;
    int64_t blk_bytes;
    uint32_t off[NI];
    int dst[NI];  // chunk index of the instruction's destination within a stage, or -1 (dummy)
    int chunk;
    // ROWS: the operand's tile rows (256 or 320)
    template <typename Id>
    __device__ __forceinline__ void init(const T* src, int64_t ld, int64_t mn0, int64_t mn_lim, int stage_off,
                                         const Id& id) {
        constexpr int rows = ROWS;
        const int64_t row_ld = BLK ? 256 : LAY == kTiled ? 4 * VEC : ld;
        if constexpr (BLK) {
            base = (const char*)uniform_ptr(src + mn0 * 256);
            blk_bytes = ld * 256 * (int64_t)sizeof(T);
        } else if constexpr (LAY == kTiled) {
            rsrc = make_rsrc(src + (mn0 / rows) * ld * (rows * 4 * VEC));
        } else {
            rsrc = make_rsrc(src + mn0 * ld);
        }
        chunk = (id.lane & 3) ^ (((id.lane >> 4) ^ (id.lane >> 3)) & 3);
#pragma unroll
        for (int t = 0; t < NI; ++t) {
            const int g = 8 * t + id.w;  // 16-row group
            const int row = 16 * g + (id.lane >> 2);
            const bool real = 16 * g < rows;
            off[t] = real && mn0 + row < mn_lim ? (uint32_t)((row * row_ld + chunk * VEC) * (int64_t)sizeof(T)) : kOOB;
            dst[t] = real ? stage_off + 64 * g : -1;
        }
    }
    template <typename Id>
    __device__ __forceinline__ void issue_one(u32x4* L, int stage, int t, int64_t k0, int64_t k_lim, bool full,
                                              bool live, const Id& id) const {
        // off[t] is already out of range for a dummy instruction's lanes
        const bool in = live && (full || (int64_t)chunk * VEC < k_lim - k0);
        u32x4* d = dst[t] >= 0 ? L + stage * WST + dst[t] : L + 4 * WST + 64 * (id.w & 3);
        if constexpr (BLK) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (k0 >> 8) * blk_bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)d, 16, (int)(in ? off[t] : kOOB),
                                                     (int)((k0 & 255) * (int64_t)sizeof(T)), 0, 0);
        } else if constexpr (LAY == kTiled) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)d, 16, (int)(in ? off[t] : kOOB),
                                                     (int)((k0 / (4 * VEC)) * (ROWS * 64)), 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)d, 16, (int)(in ? off[t] : kOOB),
                                                     (int)(k0 * (int64_t)sizeof(T)), 0, 0);
        }
    }
};

// An M/N-contiguous bf16 operand of the wide tile (kTrans). A stage holds its 32 K rows as
// blocks of 32 columns, 2 KB each: [K half ks][16 rows][64 bytes], the half ks holding the K
// indices 8g + 4ks + r (g, r = 0..3) as row 4g + r. Each DMA instruction fills one half of one
// block, four lanes a 64-byte source row, so eight consecutive lanes read one whole 128-byte
// line of a row pair. ds_read_b64_tr_b16 (gfx950) reads a 4 x 16 block of 16-bit values per
// group of 16 lanes, lanes 4r .. 4r+3 supplying row r and lane j receiving column j (checked on
// hardware); two such reads give a lane the 8 consecutive K values of its column that a
// 16 x 16 x 32 MFMA operand needs. Plain 8-byte reads cost the loop about 19 % against the
// 16-byte reads of K-contiguous operands, the transpose about 5 % more, so this mode serves the
// paths that keep no transposed copy (the memory-lean backward).
template <int NI, int ROWS, bool TILED = false>
struct KOperandTR {
    const bf16_t* src;  // the tile's first column (kTrans: element (k, j) at src[k * ld + j])
    int64_t ld;
    uint32_t voff[NI];
    int dst[NI];  // chunk index of the destination within a stage, or -1 (dummy)
    int kk[NI];   // the lane's K row within the stage
    bool ok[NI];
    template <typename P, typename Id>
    __device__ __forceinline__ void init(const P* s, int64_t ld_, int64_t mn0, int64_t mn_lim, int stage_off,
                                         const Id& id) {
        src = (const bf16_t*)s;
        ld = ld_;
        const int rs = id.lane >> 2, c = id.lane & 3, g = rs >> 2, r = rs & 3;
#pragma unroll
        for (int t = 0; t < NI; ++t) {
            const int idx = 8 * t + id.w;  // instruction: block idx/2, K half idx%2
            const bool real = idx < 2 * (ROWS / 32);
            const int b = idx >> 1, ks = idx & 1;
            const int k = 8 * g + 4 * ks + r, j = 32 * b + 8 * c;
            voff[t] = TILED ? (uint32_t)((b * 8192 + k * 32 + 8 * c) * 2) : (uint32_t)(((int64_t)k * ld + j) * 2);
            kk[t] = k;
            ok[t] = real && mn0 + j < mn_lim;
            dst[t] = real ? stage_off + (2 * b + ks) * 64 : -1;
        }
    }
    template <typename Id>
    __device__ __forceinline__ void issue_one(u32x4* L, int stage, int t, int64_t k0, int64_t k_lim, bool, bool live,
                                              const Id& id) const {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(TILED ? src + ((k0 >> 8) * ld * 8192 + (k0 & 255) * 32) : src + k0 * ld);
        const bool in = live && ok[t] && k0 + kk[t] < k_lim;
        u32x4* d = dst[t] >= 0 ? L + stage * WST + dst[t] : L + 4 * WST + 64 * (id.w & 3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)d, 16, (int)(in ? voff[t] : kOOB), 0, 0, 0);
    }
};

typedef short kd_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) kd_v4s lds_v4s;

// The MFMA operand of 16-column group c16 of a kTrans operand stage: lane l gets column l%16
// at K 8*(l/16) .. +7.
__device__ __forceinline__ u32x4 trfrag(const u32x4* S, int c16, int lane) {
    const int b = c16 >> 1, h = c16 & 1, g = lane >> 4, x = lane & 15;
    const char* p = (const char*)S + b * 2048 + (4 * g + (x >> 2)) * 64 + h * 32 + (x & 3) * 8;
    const kd_v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const kd_v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 1024));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 a = __builtin_bit_cast(u2, r1), c = __builtin_bit_cast(u2, r2);
    return u32x4{a[0], a[1], c[0], c[1]};
}

// Wide tile on 16 x 16 blocks: eight waves in a 2 x 4 grid, 128 x 80 per wave = 8 x 5 blocks,
// acc[i][j] at tile rows wm*128 + 16i, columns wn*80 + 16j (WaveIdN<8>). The stage layout and
// DMA are those above; the schedule is gemm_tile_kk16's: part 0 = A rows 0-3 while A rows 4-7
// of the stage are read, barrier, part 1 = A rows 4-7 with the DMA of stage k+4 and the reads of
// stage k+1 (A rows 0-3, and B into the other of two register sets).
template <typename T, int BA = kRow, int BB = kRow>
__device__ __forceinline__ void gemm_tile_w16(f32x4 (&acc)[8][5], u32x4* L, const WaveIdN<8>& id, const T* A,
                                              int64_t lda, int64_t m0, int64_t m_lim, int64_t ka_lim, const T* B,
                                              int64_t ldb, int64_t n0, int64_t n_lim, int64_t kb_lim, int64_t k_begin,
                                              int64_t k_end) {
    constexpr int BKH = Elem<T>::BK / 2;
    constexpr int MM = Mfma16Count<T>::N;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = (int)((k_end - k_begin + BKH - 1) / BKH);
    if (nk <= 0) return;
    constexpr bool TA = BA == kTrans || BA == kTransT, TB = BB == kTrans || BB == kTransT;
    static_assert((!TA && !TB) || sizeof(T) == 2, "kTrans and kTransT operands are bf16");
    typename std::conditional<TA, KOperandTR<2, kTileM, BA == kTransT>, KOperandW<T, BA, 2, kTileM>>::type opA;
    typename std::conditional<TB, KOperandTR<3, kWideN, BB == kTransT>, KOperandW<T, BB, 3, kWideN>>::type opB;
    opA.init(A, lda, m0, m_lim, 0, id);
    opB.init(B, ldb, n0, n_lim, kTileM * NCH4, id);
    auto kof = [&](int s) { return k_begin + (int64_t)s * BKH; };
    auto issue = [&](int s) {
        const bool live = s < nk;
        const bool fa = kof(s) + BKH <= ka_lim, fb = kof(s) + BKH <= kb_lim;
#pragma unroll
        for (int t = 0; t < 2; ++t) opA.issue_one(L, s & 3, t, kof(s), ka_lim, fa, live, id);
#pragma unroll
        for (int t = 0; t < 3; ++t) opB.issue_one(L, s & 3, t, kof(s), kb_lim, fb, live, id);
    };
    u32x4 fa[8], fb[2][5];
    auto rdA = [&](int i0, int s) {
        const u32x4* S = L + (s & 3) * WST;
#pragma unroll
        for (int i = i0; i < i0 + 4; ++i)
            fa[i] = TA ? trfrag(S, id.wm * 8 + i, id.lane) : frag16(S, id.wm * 128 + 16 * i, id.lane);
    };
    auto rdB = [&](u32x4 (&b)[5], int s) {
        const u32x4* S = L + (s & 3) * WST + kTileM * NCH4;
#pragma unroll
        for (int j = 0; j < 5; ++j)
            b[j] = TB ? trfrag(S, id.wn * 5 + j, id.lane) : frag16(S, id.wn * 80 + 16 * j, id.lane);
    };
    // LDS reads per fragment: two for a kTrans operand
    constexpr int RA = TA ? 2 : 1, RB = TB ? 2 : 1;
    constexpr int NRD1 = 4 * RA + 5 * RB;                 // reads under part 1's 15 MFMAs
    constexpr int RDG = NRD1 <= 15 ? NRD1 : (NRD1 + 1) / 2, RDPER = NRD1 <= 15 ? 1 : 2;
    auto stage = [&](int k, const u32x4 (&bc)[5], u32x4 (&bn)[5], bool more) {
        KD_SCHED_FENCE();
        rdA(4, k);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 5; ++j) mma16<T>(acc[i][j], fa[i], bc[j]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 4 * MM, 0);
            __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, RA, 0);
        }
        __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 4 * MM, 0);
        KD_SCHED_FENCE();
        if (more)
            wait_vmem_le<10>();  // stage k+1 complete; k+2 and k+3 may be in flight
        else
            wait_vmem_le<0>();
        lds_barrier();
        KD_SCHED_FENCE();
        if (more) {
            issue(k + 4);
            rdA(0, k + 1);
            rdB(bn, k + 1);
        }
#pragma unroll
        for (int i = 4; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 5; ++j) mma16<T>(acc[i][j], fa[i], bc[j]);
        if (more) {
            // 20 MFMAs carry 5 DMA issues and the fragment reads (9 from K-contiguous operands)
#pragma unroll
            for (int q = 0; q < 5; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, MM, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_VMEM_RD, 1, 1);
            }
#pragma unroll
            for (int q = 0; q < RDG; ++q) {
                __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, MM, 1);
                __builtin_amdgcn_sched_group_barrier(KD_SG_DS_RD, RDPER, 1);
            }
            __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, (15 - RDG) * MM, 1);
        }
        KD_SCHED_FENCE();
    };
    // five DMA instructions per wave per stage
#pragma unroll
    for (int s = 0; s < 4; ++s) issue(s);
    wait_vmem_le<15>();
    lds_barrier();
    rdA(0, 0);
    rdB(fb[0], 0);
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
        stage(kt, fb[0], fb[1], true);
        stage(kt + 1, fb[1], fb[0], true);
    }
    stage(kt, fb[0], fb[1], kt + 1 < nk);
    if (kt + 1 < nk) stage(kt + 1, fb[1], fb[0], false);
    wait_vmem_le<0>();  // no zero-fill may land after the caller reuses the LDS
    __syncthreads();
}

// Workgroups go to the 8 XCDs round robin (id % 8). Give XCD x the contiguous range
// [x*per, (x+1)*per) of logical tiles, in dispatch order, so tiles that share operands run
// on the same L2 at about the same time. Returns n (no work) for the padding ids.
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t n) {
    const int64_t per = (n + 7) / 8;
    const int64_t t = (id % 8) * per + id / 8;
    return t < n ? t : n;
}

__device__ __forceinline__ int acc_row(int i, int e, int h) { return i * 32 + 8 * (e >> 2) + 4 * h + (e & 3); }

}  // namespace kdkl
