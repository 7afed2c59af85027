// C ABI of libkdkl (declared in include/kdkl.h): argument checks, workspace layout and the
// order of kernel launches. All arithmetic lives in kdkl_kernels.hip.
//
// Orchestration follows the pages' fused chunked KL loss ("Making knowledge distillation
// cheap enough to run in production", paragraph on the second fix):
//   forward   one pass over all rows. Every 256 x 256 logit tile lives in registers only;
//             it is folded into per-row running (max, sum) partials and the gather of the
//             cached ids, then dropped.
//   backward  one pass per chunk of rows. Recompute the chunk's logit tiles, form the
//             gradient tile G_c [chunk, V] in the workspace, then dH = G_c W for those rows
//             and dW += G_c^T H_c.
// So peak memory depends on the sequence only through H, dH and the O(N*K) cache terms.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "kdkl.h"
#include "kdkl_internal.h"

using namespace kdkl;

// Device scratch of kd_fused_kl_fwd_noalloc: the forward's workspace for callers that cannot
// allocate. Every GPU the library runs on holds its own copy until the process ends. Host code
// never passes this name to a kernel or a copy (on the host it is only a stand-in for the
// symbol); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxD = (int64_t)1 << 20;  // keeps a tile's 256 rows of d fp32 within 32-bit offsets
// Chunks per dW pass: as many as make about 8192 tokens (4 chunks of 2048). Each pass reads and
// writes all of dW once, so few tokens per pass multiply that traffic; many make each
// vocabulary tile's G^T slab outgrow the L2 (16384 tokens measured 4% slower than 8192, and 4096
// tokens 6% slower). It depends on the chunk only, so the workspace does not grow with N; a
// group the batch does not fill ends with the last chunk.
constexpr int64_t kDwTokens = 8192;
// K columns per chunk in G_c^T and H_c^T: whole 32-column stages of the stage-tiled layout, the
// columns past the chunk's rows zero.
int64_t slot_cols(int64_t C) { return round_up(C, 32); }
int64_t dw_group(const kd_problem*, int64_t C) { return std::max<int64_t>(1, kDwTokens / slot_cols(C)); }

struct Carve {
    uintptr_t base;
    size_t used = 0;
    explicit Carve(void* p) : base((uintptr_t)p) {}
    void* take(size_t bytes) {
        used = (size_t)round_up((int64_t)used, kAlign);
        void* p = (void*)(base + used);
        used += bytes;
        return p;
    }
};

int64_t n_vtiles(int64_t V) { return (V + kTileN - 1) / kTileN; }
int64_t n_rblocks(int64_t rows) { return (rows + kTileM - 1) / kTileM; }
size_t esize(int32_t dt) { return dt == KD_BF16 ? 2 : 4; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Host-side checks; nothing is enqueued before they pass.
kd_status check_problem(const kd_problem* p) {
    if (!p) return KD_ERR_NULL;
    if (p->act != KD_FP32 && p->act != KD_BF16) return KD_ERR_DTYPE;
    if (p->tlogit != KD_FP32 && p->tlogit != KD_BF16) return KD_ERR_DTYPE;
    if (p->N < 1 || p->d < 8 || p->d % 8 != 0 || p->d > kMaxD || p->V < 1 || p->V > (int64_t)kTileN * kMaxVTiles) return KD_ERR_SHAPE;
    if (p->K < 1 || p->K > kMaxK || p->K > p->V || p->chunk < 1) return KD_ERR_SHAPE;
    const int64_t lim = (int64_t)1 << 31;
    if ((p->N + kTileM) * p->K >= lim || p->N * p->d >= lim || p->V * p->d >= lim) return KD_ERR_SHAPE;
    if (!std::isfinite(p->T) || !(p->T > 0.f)) return KD_ERR_VALUE;
    if (!std::isfinite(p->n_norm)) return KD_ERR_VALUE;
    if ((p->flags & ~(KD_VALIDATE_IDX | KD_ACCUMULATE_DW | KD_SKIP_DW | KD_LOW_MEMORY)) != 0 || p->reserved != 0)
        return KD_ERR_VALUE;
    if ((p->flags & KD_SKIP_DW) && (p->flags & KD_ACCUMULATE_DW)) return KD_ERR_VALUE;
    return KD_OK;
}

Shape make_shape(const kd_problem* p) {
    Shape s;
    s.N = p->N;
    s.d = p->d;
    s.V = p->V;
    s.K = p->K;
    s.T = p->T;
    s.n_norm = p->n_norm > 0.f ? p->n_norm : (float)p->N;
    s.act = p->act == KD_BF16 ? Dt::BF16 : Dt::F32;
    s.tlog = p->tlogit == KD_BF16 ? Dt::BF16 : Dt::F32;
    return s;
}

// Rows per chunk: the caller's chunk, at most N and at most 2^20. G_c^T and H_c^T have a row
// stride of max(8192, chunk) elements and the dW product reads 320 of their rows per tile
// through 32-bit buffer offsets: 320 * 2^20 * 4 bytes stays below the descriptor range.
constexpr int64_t kMaxChunk = (int64_t)1 << 20;
int64_t chunk_rows(const kd_problem* p) { return std::min({p->chunk, p->N, kMaxChunk}); }
// The dense grids have a row stride of 4 * Vp bytes (fp32 Z, or bf16 G at twice the element
// stride), and a 256-row tile of them is read through 32-bit buffer offsets.
constexpr int64_t kMaxDenseV = (int64_t)1 << 21;
bool whole_plan(const kd_problem* p) { return chunk_rows(p) % kTileM == 0; }

// Workspace of the fused calls. The forward and backward parts are disjoint in time, so they
// overlap in the workspace; the query returns the larger of the two.
struct FusedWs {
    int32_t* plan_off;
    uint32_t* plan_ent;
    float2* part;
    float* zk;
    double* blk_sum;
    uint32_t* status;
    // backward
    int32_t* cplan_off;
    uint32_t* cplan_ent;
    float* pt;
    void* Gc;   // stage-tiled (K-blocked [Vp/256][cc][256] in the fp32 memory-lean backward)
    void* GT;   // G_c^T stage-tiled, ldgt K columns: a group of chunks side by side
    void* WT;   // W^T stage-tiled, Vp K columns, entries past V zero
    void* HT;   // H_c^T stage-tiled, ldgt K columns
    float* dh_part;
    int64_t ldgt, group;
    int n_split;
    // stage-tiled copies of W and of one row chunk of H for the forward and gradient kernels
    // (null: they read W and H as stored)
    void* Wt;
    void* Ht;   // kFwdRows rows
    void* cWt;  // the backward's
    void* cHt;  // one chunk of rows
    int64_t tS;  // stages per row block
    size_t fwd_bytes, bwd_bytes;
};

// Rows per forward launch when H is read from a stage-tiled copy: the copy holds this many rows,
// so the workspace stays independent of N. 16384 rows are 64 row blocks, which with 4 vocabulary
// lanes give each of 256 compute units one unit of work (0.3 ms per step faster than 8192 rows at
// the gpt-oss head: half the launch tails).
constexpr int64_t kFwdRows = 16384;
int64_t fwd_rows(const kd_problem* p) { return std::min(p->N, kFwdRows); }
int fwd_parts(const kd_problem* p) {
    // per-row partials of the largest launch (the last may be shorter and use more lanes)
    const int64_t F = fwd_rows(p), last = p->N - (p->N - 1) / F * F;
    return (int)std::max(2 * fwd_vsplits(F, p->V) * F, 2 * fwd_vsplits(last, p->V) * last);
}

bool low_memory(const kd_problem* p) { return (p->flags & KD_LOW_MEMORY) != 0; }

// The wide dH tile reads W^T stage-tiled in blocks of 320 rows through one buffer descriptor
// per tile: its last stage sits (Vp/SW - 1) * 320 * 64 bytes past the tile's first, which must
// stay inside the descriptor's 32-bit range (an offset past it reads zero). That caps V at
// 3,355,392 (bf16) or 1,677,568 (fp32) on every path that computes dH this way (all backward
// paths but the memory-lean one); G_c's 256-row blocks allow more.
constexpr int64_t kDescRange = 0x7FFFFFF0;
bool wide_dh_fits(const kd_problem* p) {
    const int64_t Vp = round_up(p->V, kTileN), sw = 64 / (int64_t)esize(p->act);
    return (Vp / sw) * 320 * 64 - 16 < kDescRange;
}
// The bf16 memory-lean backward's dH reads the stage-tiled G_c (256-row blocks) the same way:
// V up to 4,194,048.
bool lean_dh_fits(const kd_problem* p) {
    const int64_t Vp = round_up(p->V, kTileN), sw = 64 / (int64_t)esize(p->act);
    return p->act != KD_BF16 || (Vp / sw) * 256 * 64 - 16 < kDescRange;
}

// The forward and gradient kernels read W and H from stage-tiled copies (engine.h, kTiled):
// the copies cost one pass over W and H per call, and W's size plus a row chunk of H's in the
// workspace; the kernels' operand loads then fetch whole 128-byte lines, 7-11 % faster. Below
// kTileRows rows the copy of W costs more than it saves (4096 x 32000 x 1024 measured 5 %
// slower with it, 8192 x 151936 x 2048 5 % faster). The memory-lean backward keeps none.
constexpr int64_t kTileRows = 8192;
bool tiled_fwd(const kd_problem* p) { return !low_memory(p) && p->N >= kTileRows; }
bool tiled_bwd(const kd_problem* p) { return tiled_fwd(p); }

FusedWs layout_fused(const kd_problem* p, void* ws, bool fwd_tiles = true) {
    FusedWs w{};
    const int64_t N = p->N, K = p->K, V = p->V, d = p->d;
    const int64_t n_vt = n_vtiles(V), Vp = n_vt * kTileN;
    const int64_t C = chunk_rows(p);
    const bool lean = low_memory(p);
    // dH on the wide tile except in the fp32 memory-lean backward (bf16 lean: stage-tiled G_c, W as stored)
    w.n_split = dh_splits(C, d, V, !lean || p->act == KD_BF16);
    Carve f(ws);
    w.status = (uint32_t*)f.take(kAlign);
    w.plan_off = (int32_t*)f.take(sizeof(int32_t) * n_rblocks(N) * (n_vt + 1));
    w.plan_ent = (uint32_t*)f.take(sizeof(uint32_t) * n_rblocks(N) * kTileM * K);
    const bool ft = fwd_tiles && tiled_fwd(p);
    w.part = (float2*)f.take(sizeof(float2) * fwd_parts(p));
    w.zk = (float*)f.take(sizeof(float) * N * K);
    w.blk_sum = (double*)f.take(sizeof(double) * ((N + fwd_rows(p) - 1) / fwd_rows(p)) * combine_blocks(fwd_rows(p)));
    const Dt act = p->act == KD_BF16 ? Dt::BF16 : Dt::F32;
    w.tS = tiled_stages(act, d);
    if (ft) {
        w.Wt = f.take(tiled_bytes(act, V, d));
        w.Ht = f.take(tiled_bytes(act, fwd_rows(p), d));
    }
    w.fwd_bytes = f.used;
    Carve b(ws);
    b.take(kAlign);  // status word shared with the forward layout
    // When chunks start on row-block boundaries one plan over all N rows serves every chunk;
    // otherwise each chunk builds its own.
    const int64_t plan_rows = whole_plan(p) ? N : C;
    w.cplan_off = (int32_t*)b.take(sizeof(int32_t) * n_rblocks(plan_rows) * (n_vt + 1));
    w.cplan_ent = (uint32_t*)b.take(sizeof(uint32_t) * n_rblocks(plan_rows) * kTileM * K);
    w.pt = (float*)b.take(sizeof(float) * N * K);
    w.Gc = b.take(esize(p->act) * round_up(C, kTileM) * Vp);
    if (!lean) {
        // G_c^T and H_c^T hold a group of chunks side by side (slot s at columns
        // s*round_up(C, 8)), so one dW pass reduces over the group and dW is read and written
        // once per group. The memory-lean backward keeps none of these copies (nor W^T): dH and
        // dW read G_c, W and H as they are.
        w.group = dw_group(p, C);
        w.ldgt = w.group * slot_cols(C);
        w.GT = b.take(esize(p->act) * Vp * w.ldgt);
        w.WT = b.take(esize(p->act) * round_up(d, 320) * Vp);
        w.HT = b.take(esize(p->act) * round_up(d, 320) * w.ldgt);
    }
    w.dh_part = w.n_split > 1 ? (float*)b.take(sizeof(float) * w.n_split * C * d) : nullptr;
    if (tiled_bwd(p)) {
        w.cWt = b.take(tiled_bytes(act, V, d));
        w.cHt = b.take(tiled_bytes(act, C, d));
    }
    w.bwd_bytes = b.used;
    return w;
}

// Workspace of the two paths that keep the logits (z^T, fp32) instead of recomputing them:
//   all_rows = true   forward-chunked: z^T of all N rows, [Vp][round_up(N, 4)];
//   all_rows = false  single pass: z^T of one chunk, [Vp][round_up(C, 4)].
// The backward buffers (G_c, G_c^T, W^T, H_c^T, dH partials) are those of the fused path.
struct StoredWs {
    uint32_t* status;
    int32_t* plan_off;
    uint32_t* plan_ent;
    float* pt;
    float* zk;
    float2* part;
    double* blk_sum;
    float* zt;
    int64_t ldzt;
    void* Gc;
    void* GT;
    void* WT;
    void* HT;
    float* dh_part;
    int64_t ldgt, group;
    int n_split;
    void* Wt;   // stage-tiled W and a row chunk of H for the forward (null: as stored)
    void* Ht;
    int64_t tS;
    size_t bytes;
};

StoredWs layout_stored(const kd_problem* p, void* ws, bool all_rows) {
    StoredWs w{};
    const int64_t N = p->N, K = p->K, V = p->V, d = p->d;
    const int64_t n_vt = n_vtiles(V), Vp = n_vt * kTileN;
    const int64_t C = chunk_rows(p);
    const int64_t fwd_rows = all_rows ? N : C;
    // the forward's launches: kFwdRows rows each (forward-chunked), one chunk each (single pass)
    const int64_t F = all_rows ? std::min(N, kFwdRows) : C;
    w.n_split = dh_splits(C, d, V, true);
    w.ldzt = round_up(fwd_rows, 4);
    w.group = dw_group(p, C);
    w.ldgt = w.group * slot_cols(C);
    const int64_t n_chunks = (N + C - 1) / C;
    Carve c(ws);
    w.status = (uint32_t*)c.take(kAlign);
    w.plan_off = (int32_t*)c.take(sizeof(int32_t) * n_rblocks(N) * (n_vt + 1));
    w.plan_ent = (uint32_t*)c.take(sizeof(uint32_t) * n_rblocks(N) * kTileM * K);
    w.pt = (float*)c.take(sizeof(float) * N * K);
    w.zk = (float*)c.take(sizeof(float) * N * K);
    // Per-row partials of one forward launch; the last launch may use more vocab lanes.
    const int64_t n_launch = (N + F - 1) / F, last = N - (n_launch - 1) * F;
    const int64_t n_part_rows = std::max((int64_t)fwd_vsplits(F, V) * F, (int64_t)fwd_vsplits(last, V) * last);
    w.part = (float2*)c.take(sizeof(float2) * 2 * n_part_rows);
    w.blk_sum = (double*)c.take(sizeof(double) * n_launch * combine_blocks(F));
    w.zt = (float*)c.take(sizeof(float) * Vp * w.ldzt);
    w.Gc = c.take(esize(p->act) * round_up(C, kTileM) * Vp);
    w.GT = c.take(esize(p->act) * Vp * w.ldgt);
    w.WT = c.take(esize(p->act) * round_up(d, 320) * Vp);
    w.HT = c.take(esize(p->act) * round_up(d, 320) * w.ldgt);
    w.dh_part = w.n_split > 1 ? (float*)c.take(sizeof(float) * w.n_split * C * d) : nullptr;
    const Dt act = p->act == KD_BF16 ? Dt::BF16 : Dt::F32;
    w.tS = tiled_stages(act, d);
    if (tiled_fwd(p)) {
        w.Wt = c.take(tiled_bytes(act, V, d));
        w.Ht = c.take(tiled_bytes(act, F, d));
    }
    w.bytes = c.used;
    return w;
}

struct DenseWs {
    float* Z;
    float* P;
    int64_t ldz;
    double* row_sum;
    double* blk_sum;
    float* dh_part;
    uint32_t* status;
    int n_split;
    size_t bytes;
};

DenseWs layout_dense(const kd_problem* p, void* ws) {
    DenseWs w{};
    const int64_t N = p->N, Vp = n_vtiles(p->V) * kTileN;
    w.ldz = Vp;
    w.n_split = dh_splits(N, p->d, p->V, false);
    Carve c(ws);
    w.status = (uint32_t*)c.take(kAlign);
    w.Z = (float*)c.take(sizeof(float) * N * Vp);
    w.P = (float*)c.take(sizeof(float) * N * Vp);
    w.row_sum = (double*)c.take(sizeof(double) * N);
    w.blk_sum = (double*)c.take(sizeof(double) * ((N + 1023) / 1024));
    w.dh_part = w.n_split > 1 ? (float*)c.take(sizeof(float) * w.n_split * N * p->d) : nullptr;
    w.bytes = c.used;
    return w;
}

#define KD_TRY(x)                                  \
    do {                                           \
        if ((x) != hipSuccess) return KD_ERR_HIP;  \
    } while (0)

// The stored-logit paths' forward over rows [r0, r0 + rows): from stage-tiled copies when the
// workspace holds them (the copy of W made by the caller), as stored otherwise; same arithmetic.
kd_status stored_forward(const kd_problem* p, const Shape& sh, const StoredWs& w, const void* H, const void* W,
                         int64_t r0, int64_t rows, const int32_t* plan_off, int nvs, float* zk, float* zt,
                         hipStream_t s) {
    Shape shc = sh;
    shc.N = rows;
    const char* Hr = (const char*)H + r0 * p->d * esize(p->act);
    if (w.Wt) {
        KD_TRY(launch_tile_rows(sh.act, Hr, p->d, rows, p->d, w.Ht, s));
        KD_TRY(launch_fwd(shc, w.Ht, w.Wt, plan_off, w.plan_ent, nvs, w.part, zk, zt, w.ldzt, s, w.tS));
    } else {
        KD_TRY(launch_fwd(shc, Hr, W, plan_off, w.plan_ent, nvs, w.part, zk, zt, w.ldzt, s));
    }
    return KD_OK;
}

kd_status validate_ids(const kd_problem* p, const int32_t* idx, uint32_t* status, hipStream_t s) {
    KD_TRY(launch_validate(idx, p->N, p->K, p->V, status, s));
    uint32_t h = 0;
    KD_TRY(hipMemcpyAsync(&h, status, sizeof(h), hipMemcpyDeviceToHost, s));
    KD_TRY(hipStreamSynchronize(s));
    return h ? KD_ERR_INDEX : KD_OK;
}

// Backward over chunks from stored logits (forward-chunked path): G_c from z^T, then dH_c and
// the grouped dW passes, as in kd_fused_kl_bwd.
kd_status stored_backward(const kd_problem* p, const Shape& sh, const StoredWs& w, const void* H, const int32_t* idx,
                          const float* lse, const float* grad_loss, void* dH, float* dW, hipStream_t s) {
    const int64_t C = chunk_rows(p);
    const bool one_plan = whole_plan(p);
    const int64_t plan_stride = n_vtiles(p->V) + 1;
    const int64_t SC = slot_cols(C);
    const size_t es = esize(p->act);
    const bool acc0 = (p->flags & KD_ACCUMULATE_DW) != 0;
    int64_t ci = 0;
    bool dw_written = false;
    for (int64_t c0 = 0; c0 < p->N; c0 += C, ++ci) {
        const int64_t cc = std::min(C, p->N - c0);
        const int64_t slot = ci % w.group;
        if (!one_plan) KD_TRY(launch_plan(idx, c0, c0 + cc, p->K, p->V, w.plan_off, w.plan_ent, s));
        const int32_t* c_off = w.plan_off + (one_plan ? (c0 / kTileM) * plan_stride : 0);
        KD_TRY(launch_transpose(sh.act, (const char*)H + c0 * p->d * es, p->d, cc, p->d, w.HT, w.ldgt, slot * SC,
                                round_up(cc, 32), s));
        KD_TRY(launch_grad_z(sh, w.zt, w.ldzt, c0, lse, w.pt + c0 * p->K, grad_loss, c0, cc, c_off, w.plan_ent, w.Gc,
                             w.GT, w.ldgt, slot * SC, s));
        KD_TRY(launch_dh(sh, w.Gc, 0, nullptr, w.WT, c0, cc, w.n_split, w.dh_part, dH, s));
        if (slot == w.group - 1 || c0 + cc >= p->N) {
            KD_TRY(launch_dw_t(sh, w.GT, w.ldgt, w.HT, w.ldgt, slot * SC + cc, acc0 || dw_written, dW, s));
            dw_written = true;
        }
    }
    return KD_OK;
}

// The forward's launches, once the arguments have been checked; ws holds at least the
// forward's part of the fused workspace layout.
kd_status fused_forward(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                        float* loss, float* lse, float* row_kl, float* zk, void* ws, hipStream_t s,
                        bool tiles = true) {
    (void)hipGetLastError();  // start from a clean error state
    const Shape sh = make_shape(p);
    const FusedWs w = layout_fused(p, ws, tiles);
    if (p->flags & KD_VALIDATE_IDX) {
        const kd_status st = validate_ids(p, idx, w.status, s);
        if (st != KD_OK) return st;
    }
    float* zk_out = zk ? zk : w.zk;
    KD_TRY(launch_plan(idx, 0, p->N, p->K, p->V, w.plan_off, w.plan_ent, s));
    // Rows in launches of kFwdRows (whole row blocks), with or without stage-tiled copies (of W,
    // and of each launch's rows of H): the arithmetic, and so every result bit, is the same
    // either way. Combined per launch; the fp64 block sums line up as for one launch over all
    // rows.
    if (w.Wt) KD_TRY(launch_tile_rows(sh.act, W, p->d, p->V, p->d, w.Wt, s));
    const int64_t F = fwd_rows(p), plan_stride = n_vtiles(p->V) + 1;
    const size_t es = esize(p->act), ets = esize(p->tlogit);
    int n_blk = 0;
    for (int64_t r0 = 0; r0 < p->N; r0 += F) {
        const int64_t rows = std::min(F, p->N - r0);
        Shape shc = sh;
        shc.N = rows;
        const int nvs = fwd_vsplits(rows, p->V);
        const char* Hr = (const char*)H + r0 * p->d * es;
        if (w.Wt) {
            KD_TRY(launch_tile_rows(sh.act, Hr, p->d, rows, p->d, w.Ht, s));
            KD_TRY(launch_fwd(shc, w.Ht, w.Wt, w.plan_off + (r0 / kTileM) * plan_stride, w.plan_ent, nvs, w.part,
                              zk_out + r0 * p->K, nullptr, 0, s, w.tS));
        } else {
            KD_TRY(launch_fwd(shc, Hr, W, w.plan_off + (r0 / kTileM) * plan_stride, w.plan_ent, nvs, w.part,
                              zk_out + r0 * p->K, nullptr, 0, s));
        }
        int nb = 0;
        KD_TRY(launch_combine(shc, w.part, 2 * nvs, zk_out + r0 * p->K, (const char*)tlog + r0 * p->K * ets, lse + r0,
                              row_kl ? row_kl + r0 : nullptr, w.blk_sum + n_blk, &nb, s));
        n_blk += nb;
    }
    KD_TRY(launch_loss_final(sh, w.blk_sum, n_blk, loss, s));
    return KD_OK;
}

// Argument checks shared by the two forward entry points (nothing is enqueued).
kd_status check_forward(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                        const float* loss, const float* lse) {
    const kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    if (!H || !W || !idx || !tlog || !loss || !lse) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16)) return KD_ERR_VALUE;
    return KD_OK;
}

// Address of `scratch` on the current device, looked up once per device with that device
// current (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

kd_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KD_ERR_INTERNAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KD_ERR_HIP;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return KD_OK;
}

}  // namespace

extern "C" {

int kd_abi_version(void) { return KDKL_ABI_VERSION; }

const char* kd_status_str(kd_status s) {
    switch (s) {
        case KD_OK: return "ok";
        case KD_ERR_NULL: return "a required pointer is NULL";
        case KD_ERR_SHAPE: return "a size is out of the supported range";
        case KD_ERR_DTYPE: return "unsupported dtype";
        case KD_ERR_VALUE: return "invalid value (temperature, n_norm, flags, reserved or alignment)";
        case KD_ERR_WORKSPACE: return "workspace too small or misaligned";
        case KD_ERR_INDEX: return "a cached token id is out of range or repeated within a row";
        case KD_ERR_HIP: return "the HIP runtime reported an error";
        case KD_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

size_t kd_fused_workspace_bytes(const kd_problem* p) {
    if (check_problem(p) != KD_OK) return 0;
    const FusedWs w = layout_fused(p, nullptr);
    return std::max(w.fwd_bytes, w.bwd_bytes);
}

size_t kd_dense_workspace_bytes(const kd_problem* p) {
    if (check_problem(p) != KD_OK || p->V > kMaxDenseV) return 0;
    return layout_dense(p, nullptr).bytes;
}

kd_status kd_fused_kl_fwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                          float* loss, float* lse, float* row_kl, float* zk, void* ws, size_t ws_bytes,
                          kd_stream stream) {
    const kd_status st = check_forward(p, H, W, idx, tlog, loss, lse);
    if (st != KD_OK) return st;
    if (!ws) return KD_ERR_NULL;
    if (!aligned(ws, kAlign) || ws_bytes < kd_fused_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    return fused_forward(p, H, W, idx, tlog, loss, lse, row_kl, zk, ws, (hipStream_t)stream);
}

kd_status kd_fused_kl_fwd_noalloc(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                                  const void* tlog, float* loss, float* lse, float* row_kl, float* zk,
                                  kd_stream stream) {
    kd_status st = check_forward(p, H, W, idx, tlog, loss, lse);
    if (st != KD_OK) return st;
    // KD_VALIDATE_IDX copies a status word to the host and waits for it; kd_validate_ids is the
    // check that needs neither.
    if (p->flags & KD_VALIDATE_IDX) return KD_ERR_VALUE;
    if (layout_fused(p, nullptr, false).fwd_bytes > KD_NOALLOC_SCRATCH_BYTES) return KD_ERR_WORKSPACE;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != KD_OK) return st;
    return fused_forward(p, H, W, idx, tlog, loss, lse, row_kl, zk, ws, (hipStream_t)stream, false);
}

kd_status kd_fused_kl_bwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                          const float* lse, const float* grad_loss, void* dH, float* dW, void* ws, size_t ws_bytes,
                          kd_stream stream) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    const bool want_dw = (p->flags & KD_SKIP_DW) == 0;
    if (low_memory(p) ? !lean_dh_fits(p) : !wide_dh_fits(p)) return KD_ERR_SHAPE;
    if (!H || !W || !idx || !tlog || !lse || !dH || (want_dw && !dW) || !ws) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || (want_dw && !aligned(dW, 16))) return KD_ERR_VALUE;
    if (!aligned(ws, kAlign) || ws_bytes < kd_fused_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const Shape sh = make_shape(p);
    const FusedWs w = layout_fused(p, ws);
    if (p->flags & KD_VALIDATE_IDX) {
        st = validate_ids(p, idx, w.status, s);
        if (st != KD_OK) return st;
    }
    const int64_t C = chunk_rows(p);
    const int64_t Vp = n_vtiles(p->V) * kTileN;
    const bool acc0 = (p->flags & KD_ACCUMULATE_DW) != 0;
    const bool lean = low_memory(p);
    // W^T once per call: dH = G_c W then reads both operands with the vocabulary contiguous. The
    // same loads give the gradient kernel's stage-tiled W; each chunk's rows of H are tiled before
    // its gradient kernel.
    if (!lean) KD_TRY(launch_transpose(sh.act, W, p->d, p->V, p->d, w.WT, Vp, 0, Vp, s, w.cWt));
    const int64_t SC = slot_cols(C);
    const size_t es = esize(p->act);
    const bool one_plan = whole_plan(p);
    const int64_t plan_stride = n_vtiles(p->V) + 1;
    if (one_plan) KD_TRY(launch_plan(idx, 0, p->N, p->K, p->V, w.cplan_off, w.cplan_ent, s));
    KD_TRY(launch_teacher_prob(tlog, sh.tlog, 0, p->N, p->K, p->T, w.pt, s));
    int64_t ci = 0;
    bool dw_written = false;
    for (int64_t c0 = 0; c0 < p->N; c0 += C, ++ci) {
        const int64_t cc = std::min(C, p->N - c0);
        const int64_t slot = ci % w.group;
        if (!one_plan) KD_TRY(launch_plan(idx, c0, c0 + cc, p->K, p->V, w.cplan_off, w.cplan_ent, s));
        // The chunk's row blocks in the plan; entry offsets in it are absolute.
        const int32_t* c_off = w.cplan_off + (one_plan ? (c0 / kTileM) * plan_stride : 0);
        if (lean) {
            // G_c only (stage-tiled for bf16, K-blocked for fp32); dH reads W as stored and dW reads
            // G_c and H_c as they are.
            KD_TRY(launch_bwd_grad(sh, H, W, lse, w.pt + c0 * p->K, grad_loss, c0, cc, c_off, w.cplan_ent, w.Gc,
                                   p->act == KD_BF16, nullptr, 0, 0, s));
            KD_TRY(launch_dh(sh, w.Gc, 0, W, nullptr, c0, cc, w.n_split, w.dh_part, dH, s, true));
            if (want_dw) {
                KD_TRY(launch_dw(sh, w.Gc, 0, H, c0, cc, acc0 || dw_written, dW, s, true));
                dw_written = true;
            }
            continue;
        }
        // H_c^T into its slot, so that dW = G^T H reads both operands with the rows contiguous.
        // For whole row blocks the same loads also write the chunk's stage-tiled copy of H_c.
        const char* Hc = (const char*)H + c0 * p->d * es;
        const bool one_pass = want_dw && w.cHt && cc % kTileM == 0;
        if (want_dw)
            KD_TRY(launch_transpose(sh.act, Hc, p->d, cc, p->d, w.HT, w.ldgt, slot * SC, round_up(cc, 32), s,
                                    one_pass ? w.cHt : nullptr));
        // Without dW, G^T is not needed: the gradient kernel skips those stores.
        if (w.cHt && !one_pass) KD_TRY(launch_tile_rows(sh.act, Hc, p->d, cc, p->d, w.cHt, s));
        KD_TRY(launch_bwd_grad(sh, w.cHt ? w.cHt : H, w.cWt ? w.cWt : W, lse, w.pt + c0 * p->K, grad_loss, c0, cc,
                               c_off, w.cplan_ent, w.Gc, true, want_dw ? w.GT : nullptr, w.ldgt, slot * SC, s,
                               w.cWt ? w.tS : 0));
        KD_TRY(launch_dh(sh, w.Gc, 0, W, w.WT, c0, cc, w.n_split, w.dh_part, dH, s));
        // One dW pass per group of chunks (K = the group's rows; each slot zero-padded to 32)
        if (want_dw && (slot == w.group - 1 || c0 + cc >= p->N)) {
            KD_TRY(launch_dw_t(sh, w.GT, w.ldgt, w.HT, w.ldgt, slot * SC + cc, acc0 || dw_written, dW, s));
            dw_written = true;
        }
    }
    return KD_OK;
}

kd_status kd_dense_kl(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                      const float* grad_loss, float* loss, float* lse, float* row_kl, void* dH, float* dW, void* ws,
                      size_t ws_bytes, kd_stream stream) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    // only the fused backward can leave dW out or run memory-lean
    if (p->flags & (KD_SKIP_DW | KD_LOW_MEMORY)) return KD_ERR_VALUE;
    if (p->V > kMaxDenseV) return KD_ERR_SHAPE;
    if (!H || !W || !idx || !tlog || !loss || !lse || !dH || !dW || !ws) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16)) return KD_ERR_VALUE;
    if (!aligned(ws, kAlign) || ws_bytes < kd_dense_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const Shape sh = make_shape(p);
    const DenseWs w = layout_dense(p, ws);
    if (p->flags & KD_VALIDATE_IDX) {
        st = validate_ids(p, idx, w.status, s);
        if (st != KD_OK) return st;
    }
    KD_TRY(launch_dense_logits(sh, H, W, w.Z, w.ldz, s));
    KD_TRY(launch_dense_rows(sh, w.Z, w.P, w.ldz, idx, tlog, grad_loss, lse, row_kl, w.row_sum, nullptr, 0, s));
    int n_blk = 0;
    KD_TRY(launch_sum_rows(sh, w.row_sum, w.blk_sum, &n_blk, s));
    KD_TRY(launch_loss_final(sh, w.blk_sum, n_blk, loss, s));
    // G: bf16 over the logits grid (row stride 2*Vp elements), or fp32 in the teacher grid.
    const void* G = sh.act == Dt::BF16 ? (const void*)w.Z : (const void*)w.P;
    const int64_t ldg = sh.act == Dt::BF16 ? 2 * w.ldz : w.ldz;
    KD_TRY(launch_dh(sh, G, ldg, W, nullptr, 0, p->N, w.n_split, w.dh_part, dH, s));
    KD_TRY(launch_dw(sh, G, ldg, H, 0, p->N, (p->flags & KD_ACCUMULATE_DW) != 0, dW, s));
    return KD_OK;
}

kd_status kd_validate_ids(const int32_t* idx, int64_t N, int64_t K, int64_t V, uint32_t* status,
                          kd_stream stream) {
    if (!idx || !status) return KD_ERR_NULL;
    if (N < 1 || N > 0x7FFFFFFF || K < 1 || K > kMaxK || V < 1) return KD_ERR_SHAPE;
    (void)hipGetLastError();
    KD_TRY(launch_validate(idx, N, K, V, status, (hipStream_t)stream));
    return KD_OK;
}

kd_status kd_topk_cache(const void* logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, int64_t K,
                        int32_t* idx, void* values, kd_stream stream) {
    if (!logits || !idx || !values) return KD_ERR_NULL;
    if (dtype != KD_FP32 && dtype != KD_BF16) return KD_ERR_DTYPE;
    if (N < 1 || N > 0x7FFFFFFF || V < 1 || V > kMaxTopV || K < 1 || K > V || K > kMaxTopK || ld < V)
        return KD_ERR_SHAPE;
    const size_t es = esize(dtype);
    if (!aligned(logits, es) || !aligned(values, es) || !aligned(idx, 4)) return KD_ERR_VALUE;
    (void)hipGetLastError();
    KD_TRY(launch_topk(dtype == KD_BF16 ? Dt::BF16 : Dt::F32, logits, ld, N, V, K, idx, values, (hipStream_t)stream));
    return KD_OK;
}

size_t kd_chunked_workspace_bytes(const kd_problem* p) {
    if (check_problem(p) != KD_OK) return 0;
    return layout_stored(p, nullptr, true).bytes;
}

kd_status kd_chunked_logits(const kd_problem* p, const void* ws, size_t ws_bytes, const float** zt,
                            int64_t* ldzt) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    if (!ws || !zt || !ldzt) return KD_ERR_NULL;
    if (!aligned(ws, kAlign) || ws_bytes < kd_chunked_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    const StoredWs w = layout_stored(p, const_cast<void*>(ws), true);
    *zt = w.zt;
    *ldzt = w.ldzt;
    return KD_OK;
}

size_t kd_fused_fwdbwd_workspace_bytes(const kd_problem* p) {
    if (check_problem(p) != KD_OK) return 0;
    return layout_stored(p, nullptr, false).bytes;
}

kd_status kd_chunked_kl(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                        const float* grad_loss, float* loss, float* lse, float* row_kl, void* dH, float* dW, void* ws,
                        size_t ws_bytes, kd_stream stream) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    // only the fused backward can leave dW out or run memory-lean
    if (p->flags & (KD_SKIP_DW | KD_LOW_MEMORY)) return KD_ERR_VALUE;
    if (!wide_dh_fits(p)) return KD_ERR_SHAPE;
    if (!H || !W || !idx || !tlog || !loss || !lse || !dH || !dW || !ws) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16)) return KD_ERR_VALUE;
    if (!aligned(ws, kAlign) || ws_bytes < kd_chunked_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const Shape sh = make_shape(p);
    const StoredWs w = layout_stored(p, ws, true);
    if (p->flags & KD_VALIDATE_IDX) {
        st = validate_ids(p, idx, w.status, s);
        if (st != KD_OK) return st;
    }
    // Forward over all rows in launches of kFwdRows, keeping every logit (z^T) for the backward.
    KD_TRY(launch_plan(idx, 0, p->N, p->K, p->V, w.plan_off, w.plan_ent, s));
    KD_TRY(launch_teacher_prob(tlog, sh.tlog, 0, p->N, p->K, p->T, w.pt, s));
    if (w.Wt) KD_TRY(launch_tile_rows(sh.act, W, p->d, p->V, p->d, w.Wt, s));
    const int64_t F = std::min(p->N, kFwdRows), plan_stride = n_vtiles(p->V) + 1;
    const size_t ets = esize(p->tlogit);
    int n_blk = 0;
    for (int64_t r0 = 0; r0 < p->N; r0 += F) {
        const int64_t rows = std::min(F, p->N - r0);
        Shape shc = sh;
        shc.N = rows;
        const int nvs = fwd_vsplits(rows, p->V);
        st = stored_forward(p, sh, w, H, W, r0, rows, w.plan_off + (r0 / kTileM) * plan_stride, nvs, w.zk + r0 * p->K,
                            w.zt + r0, s);
        if (st != KD_OK) return st;
        int nb = 0;
        KD_TRY(launch_combine(shc, w.part, 2 * nvs, w.zk + r0 * p->K, (const char*)tlog + r0 * p->K * ets, lse + r0,
                              row_kl ? row_kl + r0 : nullptr, w.blk_sum + n_blk, &nb, s));
        n_blk += nb;
    }
    KD_TRY(launch_loss_final(sh, w.blk_sum, n_blk, loss, s));
    KD_TRY(launch_transpose(sh.act, W, p->d, p->V, p->d, w.WT, n_vtiles(p->V) * kTileN, 0, n_vtiles(p->V) * kTileN, s));
    return stored_backward(p, sh, w, H, idx, lse, grad_loss, dH, dW, s);
}

kd_status kd_fused_kl_fwdbwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx, const void* tlog,
                             const float* grad_loss, float* loss, float* lse, float* row_kl, void* dH, float* dW,
                             void* ws, size_t ws_bytes, kd_stream stream) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    // only the fused backward can leave dW out or run memory-lean
    if (p->flags & (KD_SKIP_DW | KD_LOW_MEMORY)) return KD_ERR_VALUE;
    if (!wide_dh_fits(p)) return KD_ERR_SHAPE;
    if (!H || !W || !idx || !tlog || !loss || !lse || !dH || !dW || !ws) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16)) return KD_ERR_VALUE;
    if (!aligned(ws, kAlign) || ws_bytes < kd_fused_fwdbwd_workspace_bytes(p)) return KD_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const Shape sh = make_shape(p);
    const StoredWs w = layout_stored(p, ws, false);
    if (p->flags & KD_VALIDATE_IDX) {
        st = validate_ids(p, idx, w.status, s);
        if (st != KD_OK) return st;
    }
    const int64_t C = chunk_rows(p);
    const bool one_plan = whole_plan(p);
    const int64_t plan_stride = n_vtiles(p->V) + 1;
    const int64_t SC = slot_cols(C);
    const size_t es = esize(p->act), ets = esize(p->tlogit);
    const bool acc0 = (p->flags & KD_ACCUMULATE_DW) != 0;
    if (one_plan) KD_TRY(launch_plan(idx, 0, p->N, p->K, p->V, w.plan_off, w.plan_ent, s));
    KD_TRY(launch_teacher_prob(tlog, sh.tlog, 0, p->N, p->K, p->T, w.pt, s));
    KD_TRY(launch_transpose(sh.act, W, p->d, p->V, p->d, w.WT, n_vtiles(p->V) * kTileN, 0, n_vtiles(p->V) * kTileN, s));
    if (w.Wt) KD_TRY(launch_tile_rows(sh.act, W, p->d, p->V, p->d, w.Wt, s));
    int64_t ci = 0;
    int n_blk = 0;
    bool dw_written = false;
    for (int64_t c0 = 0; c0 < p->N; c0 += C, ++ci) {
        const int64_t cc = std::min(C, p->N - c0);
        const int64_t slot = ci % w.group;
        if (!one_plan) KD_TRY(launch_plan(idx, c0, c0 + cc, p->K, p->V, w.plan_off, w.plan_ent, s));
        const int32_t* c_off = w.plan_off + (one_plan ? (c0 / kTileM) * plan_stride : 0);
        // The chunk's logits, once: loss terms and z^T, which the gradient tile then reads.
        Shape shc = sh;
        shc.N = cc;
        const int nvs = fwd_vsplits(cc, p->V);
        st = stored_forward(p, sh, w, H, W, c0, cc, c_off, nvs, w.zk + c0 * p->K, w.zt, s);
        if (st != KD_OK) return st;
        int nb = 0;
        KD_TRY(launch_combine(shc, w.part, 2 * nvs, w.zk + c0 * p->K, (const char*)tlog + c0 * p->K * ets, lse + c0,
                              row_kl ? row_kl + c0 : nullptr, w.blk_sum + n_blk, &nb, s));
        n_blk += nb;
        KD_TRY(launch_transpose(sh.act, (const char*)H + c0 * p->d * es, p->d, cc, p->d, w.HT, w.ldgt, slot * SC,
                                round_up(cc, 32), s));
        KD_TRY(launch_grad_z(sh, w.zt, w.ldzt, 0, lse, w.pt + c0 * p->K, grad_loss, c0, cc, c_off, w.plan_ent, w.Gc,
                             w.GT, w.ldgt, slot * SC, s));
        KD_TRY(launch_dh(sh, w.Gc, 0, nullptr, w.WT, c0, cc, w.n_split, w.dh_part, dH, s));
        if (slot == w.group - 1 || c0 + cc >= p->N) {
            KD_TRY(launch_dw_t(sh, w.GT, w.ldgt, w.HT, w.ldgt, slot * SC + cc, acc0 || dw_written, dW, s));
            dw_written = true;
        }
    }
    KD_TRY(launch_loss_final(sh, w.blk_sum, n_blk, loss, s));
    return KD_OK;
}

}  // extern "C"
