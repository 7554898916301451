// Fused differential-attention forward on bf16 MFMA (gfx950), V1 and V2.
//
// Computes, per query row, O = softmax(s Q1 K1^T) V - lambda softmax(s Q2 K2^T) V, which equals
// (A1 - lambda A2) V exactly ("Differential Transformer: softmax can't say zero, so it subtracts",
// section "What it costs": a fused kernel computes A1 V and A2 V because the maps are never
// materialised). V1 follows "Noise-Canceling Attention by Subtraction", sections "The mechanism"
// and "Making lambda learnable and stable" (RMSNorm * (1 - lambda_init) epilogue); V2 follows
// "softmax can't say zero", section "DIFF V2: what the authors changed" (query heads 2p, 2p+1 of
// one GQA group share K and V; lambda per token and pair; no norm).
//
// Design (one pass over K/V, both maps at once):
//  - A block owns a tile of query rows of one head (V1) or of every pair of one KV group (V2).
//    Each wave owns 32 query rows of one pair. K/V tiles of 32 keys are staged through an LDS
//    ring (V1: four stages, one block barrier per pair of tiles; V2: two stages), so every tile is
//    read from memory once per block and V once for both maps.
//  - Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane (n, h)
//    then holds 16 keys of query n, so the running max and sum of each map are per-lane values
//    (one exchange between lanes n and n+32 per tile).
//  - The output is accumulated transposed, O^T += V^T P^T: P^T comes straight from the score
//    registers (rounded to bf16), V^T is read from the row-major V tile with the gfx950
//    transposing LDS read (ds_read_b64_tr_b16), so V is never transposed in registers.
//  - Online softmax per map in base 2, the scale * log2 e applied to the fp32 scores in the same
//    FMA that subtracts the running maximum (Q is used as given, so the logits carry no extra
//    rounding). The running maximum is only raised when a tile's maximum exceeds it by more than
//    8 (so unnormalised weights stay below 2^8); the final normalisation uses the same maximum,
//    so the result is unchanged.
//  - Each tile's softmax is split by key half so that the first half's MFMAs overlap the second
//    half's exponentials; V1 raises the wave priority while it issues MFMAs.
//  - Epilogue in registers: O1/l1 - lambda O2/l2, then (V1) RMSNorm over the 128 channels and the
//    (1 - lambda_init) multiply, stored as bf16.
//  - V2 (head dimension 128): the first head's Q fragments stay in registers, the second head's
//    rows sit in an LDS region of the wave's own (filled once by DMA, read with the K offsets).
//    Both in registers would need more than the 256 of two waves per SIMD, and the spill reloads
//    inside the tile loop would each wait for the whole vector-memory count, prefetch included.
#pragma once
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tile.hpp"

namespace diffattn {

// included by fwd_mfma.hip and fwd_mfma_long.hip, which build the same kernels under two
// instruction schedules: each gets its own copy
namespace {

constexpr int kBN = 32;          // keys per tile
constexpr int kDV = 128;         // value width
constexpr float kRescaleThreshold = 8.0f;

// Per-tile instruction scheduling (see the PV section): explicit MFMA / VALU interleave and
// raised wave priority while issuing MFMAs. Both help the V1 kernel (4 waves, no spills); the
// V2 kernel (8 waves of 256 registers) runs best without them.
#ifndef DA_SCHED_V1
#define DA_SCHED_V1 1
#endif
#ifndef DA_PRIO_V1
#define DA_PRIO_V1 1
#endif
#ifndef DA_SCHED_V2
#define DA_SCHED_V2 0
#endif
#ifndef DA_PRIO_V2
#define DA_PRIO_V2 0
#endif

template <int V>
struct StageC { static constexpr int value = V; };

template <int D, bool V2, bool F8 = false>
struct Cfg {
    static constexpr int NW = V2 ? 8 : 4;              // waves per block
    static constexpr int NT = NW * 64;
    static constexpr int NK = V2 ? 1 : 2;               // K tiles per stage (V2 shares K)
    static constexpr int K_ELT = F8 ? 1 : 2;            // bytes per K element (fp8 or bf16)
    static constexpr int K_CPR = D * K_ELT / 16;        // 16-byte chunks per K row
    static constexpr int V_CPR = kDV / 8;
    static constexpr int K_BYTES = kBN * D * K_ELT;
    static constexpr int V_BYTES = kBN * kDV * 2;
    static constexpr int STAGE_BYTES = NK * K_BYTES + V_BYTES;
    static constexpr int NSTAGE = V2 ? 2 : 4;                            // LDS ring (V1: two pairs of tiles)
    static constexpr int Q2_OFF = NSTAGE * STAGE_BYTES;                  // V2: Q_{2p+1} rows, per wave
    static constexpr int Q2_BYTES = V2 ? NW * 32 * D * 2 : 0;
    // DMA loads per thread per K tile; fp8: the K1 and K2 tiles together take one load per thread
    static constexpr int K_LOADS = F8 ? 1 : kBN * K_CPR / NT;
    static constexpr int V_LOADS = kBN * V_CPR / NT;
    static_assert(K_LOADS >= 1 && V_LOADS >= 1, "tile must cover every thread");
    static_assert(!F8 || (!V2 && NK * kBN * K_CPR == NT), "fp8 K tiles: one 16-byte slot per thread");
};

// fp8 K tiles (32 rows of 64 bytes): chunk c of row r at c ^ ((r >> 2) & 3), so 16 consecutive
// rows of one chunk fall on distinct banks
__device__ __forceinline__ int f8_swz(int row) { return (row >> 2) & 3; }
typedef int i32x8 __attribute__((ext_vector_type(8)));

// offset of (b, token, head)'s two maps in the [batch, seq_q, heads, 2, 128] training output
__device__ __forceinline__ int64_t row_major_maps(const MfmaFwdArgs& a, int b, int qrow, int h) {
    return (((int64_t)b * a.seq_q + qrow) * a.heads + h) * 2 * kDV;
}

template <int D, bool V2, bool CAUSAL, bool EPI, bool F8 = false, bool LAMF = false>
__global__ __launch_bounds__(V2 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(V2 ? 1 : 2, 2)))
void fwd_mfma_kernel(MfmaFwdArgs a) {
    using C = Cfg<D, V2, F8>;
    // a static allocation: its address is a compile-time constant, so each LDS operand address is a
    // lane offset plus an immediate (an extern array's base is a link-time symbol, added to every
    // address with a VALU instruction)
    __shared__ __align__(16) unsigned char smem[C::NSTAGE * C::STAGE_BYTES + C::Q2_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the tile guards are scalar
    const int lane = tid & 63;
    const int n = lane & 31;   // query column within the wave's 32 rows
    const int h2 = lane >> 5;  // which half of the MFMA k-dimension this lane feeds

    // ---- block -> (query tile, head or KV group, batch); heavy causal tiles first, and the
    //      tiles of one head kept on one XCD (blocks are dealt round-robin over 8 XCDs).
    const int pairs_per_block = V2 ? a.kv_group / 2 : 1;
    const int qsubs = C::NW / pairs_per_block;         // 32-row slices per block
    const int BM = 32 * qsubs;
    const int n_units = V2 ? a.batch * (a.heads * 2 / a.kv_group) : a.batch * a.heads;
    const int nqt = (a.seq_q + BM - 1) / BM;
    int unit, qt;
    {
        const int bid = blockIdx.x;
        // blocks resident at once on one XCD (32 CUs; two V1 blocks or one V2 block per CU)
        constexpr int kConc = 32 * (V2 ? 1 : 2);
        if ((n_units & 7) == 0) {
            const int per = n_units >> 3;
            const int slot = bid >> 3;
            if (nqt >= 2 * kConc) {
                // many query tiles per unit: chunks of kConc consecutive tiles of one unit, the
                // units' first chunks first, so the blocks resident together on an XCD mostly
                // stream the same unit's K and V (L2 reuse) while the heavy causal tiles still go
                // first
                const int c = slot / (kConc * per), within = slot % (kConc * per);
                const int cc = min(kConc, nqt - c * kConc);
                unit = (bid & 7) * per + within / cc;
                qt = c * kConc + within % cc;
            } else {
                unit = (bid & 7) * per + slot % per;
                qt = slot / per;
            }
        } else {
            unit = bid % n_units;
            qt = bid / n_units;
        }
        if (CAUSAL) qt = nqt - 1 - qt;
    }
    const int n_groups = V2 ? (a.heads * 2 / a.kv_group) : a.heads;
    const int b = unit / n_groups;
    const int grp = unit % n_groups;      // V1: head; V2: KV head
    const int pair_in_grp = wave % pairs_per_block;
    const int qsub = wave / pairs_per_block;
    const int q0 = qt * BM;
    const int qw0 = q0 + qsub * 32;       // first query row of this wave
    const int qrow = qw0 + n;
    const int off = a.seq_k - a.seq_q;    // causal alignment to the last key

    int hq1, hq2, hout, kvh;
    if (V2) {
        hout = grp * pairs_per_block + pair_in_grp;   // output pair index p
        hq1 = 2 * hout;
        hq2 = 2 * hout + 1;
        kvh = grp;
    } else {
        hout = hq1 = hq2 = kvh = grp;
    }

    // ---- Q fragments (B operand of S^T = K Q^T): lane (n, h2) holds q[n][16kk + 8h2 .. +7]
    constexpr int NKK = D / 16;
    bf16x8 bq1[NKK], bq2[NKK];
    // fp8: lane (n, h2) holds q[n][32 h2 .. +31] (the fp8 MFMA takes k = 64 in one step; A and B
    // operands use the same lane-to-k assignment, so any fixed one gives the dot product)
    i32x8 fq1 = {}, fq2 = {};
    {
        const bool ok = qrow < a.seq_q;
        const int qr = ok ? qrow : 0;
        if (F8) {
            const unsigned char* q1p = (const unsigned char*)a.q1 + b * a.q1s[0] + (int64_t)qr * a.q1s[1] +
                                       (int64_t)hq1 * a.q1s[2] + 32 * h2;
            const unsigned char* q2p = (const unsigned char*)a.q2 + b * a.q2s[0] + (int64_t)qr * a.q2s[1] +
                                       (int64_t)hq2 * a.q2s[2] + 32 * h2;
            if (ok) {
                const u32x4 x0 = *(const u32x4*)q1p, x1 = *(const u32x4*)(q1p + 16);
                const u32x4 y0 = *(const u32x4*)q2p, y1 = *(const u32x4*)(q2p + 16);
                fq1 = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                fq2 = i32x8{(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
            }
        } else {
            const bf16* q1p = (const bf16*)a.q1 + b * a.q1s[0] + (int64_t)qr * a.q1s[1] + (int64_t)hq1 * a.q1s[2] + 8 * h2;
            const bf16* q2p = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)qr * a.q2s[1] + (int64_t)hq2 * a.q2s[2] + 8 * h2;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8 z = {};
                bq1[kk] = ok ? ld_global_bf16x8(q1p + 16 * kk) : z;
                if (!V2) bq2[kk] = ok ? ld_global_bf16x8(q2p + 16 * kk) : z;
            }
        }
    }

    // ---- key range
    const int nkt_all = (a.seq_k + kBN - 1) / kBN;
    int nkt = nkt_all;
    if (CAUSAL) {
        const int qlast = min(q0 + BM, a.seq_q) - 1;
        nkt = min(nkt_all, (qlast + off) / kBN + 1);
    }
    const int wave_qlast = min(qw0 + 31, a.seq_q - 1);
    const bool wave_active = qw0 < a.seq_q;

    // ---- tile DMA: thread tid fills K slots tid + j*NT and V slots tid + j*NT of a stage.
    //      Per-lane byte offsets within a tile are fixed; the tile base advances in SGPRs.
    const bf16* kbase1 = (const bf16*)a.k1 + b * a.k1s[0] + (int64_t)kvh * a.k1s[2];
    const bf16* kbase2 = (const bf16*)a.k2 + b * a.k2s[0] + (int64_t)kvh * a.k2s[2];
    const bf16* vbase = (const bf16*)a.v + b * a.vs[0] + (int64_t)kvh * a.vs[2];
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    int krow[C::K_LOADS], kcol[C::K_LOADS], vrow[C::V_LOADS], vcol[C::V_LOADS];
    uint32_t koff1[C::K_LOADS], koff2[C::K_LOADS], voffg[C::V_LOADS];
#pragma unroll
    for (int j = 0; j < C::K_LOADS; ++j) {
        if (F8) {
            // thread tid fills slot tid % 128 of the K1 (tid < 128) or K2 tile: byte offsets
            const int s = tid & 127;
            krow[j] = s / C::K_CPR;
            kcol[j] = (s % C::K_CPR) ^ f8_swz(krow[j]);
            koff1[j] = (uint32_t)(krow[j] * a.k1s[1] + kcol[j] * 16);
            koff2[j] = (uint32_t)(krow[j] * a.k2s[1] + kcol[j] * 16);
        } else {
            const int s = tid + j * C::NT;
            krow[j] = s / C::K_CPR;
            kcol[j] = (s % C::K_CPR) ^ k_swz<D>(krow[j]);
            koff1[j] = (uint32_t)(krow[j] * a.k1s[1] + kcol[j] * 8) * 2u;
            koff2[j] = (uint32_t)(krow[j] * a.k2s[1] + kcol[j] * 8) * 2u;
        }
    }
#pragma unroll
    for (int j = 0; j < C::V_LOADS; ++j) {
        const int s = tid + j * C::NT;
        vrow[j] = s / C::V_CPR;
        vcol[j] = v_logical(vrow[j], s % C::V_CPR);
        voffg[j] = (uint32_t)(vrow[j] * a.vs[1] + vcol[j] * 8) * 2u;
    }

    auto issue_tile = [&](int kt, int stage) {
        const uint32_t st = smem_lds + stage * C::STAGE_BYTES + wave_u * 64 * 16;
        const bool full = (kt + 1) * kBN <= a.seq_k;
        const int rows_left = a.seq_k - 1 - kt * kBN;   // last valid row within this tile
        if (F8) {
            // waves 0, 1 fill the K1 tile and waves 2, 3 the K2 tile (byte addressing)
            const bool t1 = wave_u >= 2;
            const int64_t rs = t1 ? a.k2s[1] : a.k1s[1];
            const unsigned char* tb = (const unsigned char*)(t1 ? a.k2 : a.k1) + b * (t1 ? a.k2s[0] : a.k1s[0]) +
                                      (int64_t)kvh * (t1 ? a.k2s[2] : a.k1s[2]) + (int64_t)kt * kBN * rs;
            const uint32_t off = full ? (t1 ? koff2[0] : koff1[0])
                                      : (uint32_t)(min(krow[0], rows_left) * rs + kcol[0] * 16);
            dma16(tb, off, st);
        } else {
#pragma unroll
            for (int t = 0; t < C::NK; ++t) {
                const bf16* tb = (t == 0 ? kbase1 : kbase2) + (int64_t)kt * kBN * (t == 0 ? a.k1s[1] : a.k2s[1]);
                const int64_t rs = t == 0 ? a.k1s[1] : a.k2s[1];
#pragma unroll
                for (int j = 0; j < C::K_LOADS; ++j) {
                    const uint32_t off = full ? (t == 0 ? koff1[j] : koff2[j])
                                              : (uint32_t)(min(krow[j], rows_left) * rs + kcol[j] * 8) * 2u;
                    dma16(tb, off, st + t * C::K_BYTES + j * C::NT * 16);
                }
            }
        }
        const bf16* vb = vbase + (int64_t)kt * kBN * a.vs[1];
#pragma unroll
        for (int j = 0; j < C::V_LOADS; ++j) {
            const uint32_t off = full ? voffg[j] : (uint32_t)(min(vrow[j], rows_left) * a.vs[1] + vcol[j] * 8) * 2u;
            dma16(vb, off, st + C::NK * C::K_BYTES + j * C::NT * 16);
        }
    };
    // rows past the last key were fetched from a clamped address; zero them once the DMA landed
    // (only the last tile can have such rows)
    auto zero_tail = [&](int kt, int stage) {
        unsigned char* st = smem + stage * C::STAGE_BYTES;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (F8) {
            if (kt * kBN + krow[0] >= a.seq_k) *(u32x4*)(st + tid * 16) = z;
        } else {
#pragma unroll
            for (int t = 0; t < C::NK; ++t)
#pragma unroll
                for (int j = 0; j < C::K_LOADS; ++j) {
                    const int s = tid + j * C::NT;
                    if (kt * kBN + krow[j] >= a.seq_k) *(u32x4*)(st + t * C::K_BYTES + s * 16) = z;
                }
        }
#pragma unroll
        for (int j = 0; j < C::V_LOADS; ++j) {
            const int s = tid + j * C::NT;
            if (kt * kBN + vrow[j] >= a.seq_k) *(u32x4*)(st + C::NK * C::K_BYTES + s * 16) = z;
        }
    };

    // ---- per-lane LDS offsets of the MFMA operands
    // K (A operand of S^T): row n, logical chunk 2kk + h2
    int koff[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) koff[kk] = n * (D * 2) + (((2 * kk + h2) ^ k_swz<D>(n)) * 16);
    // fp8 K (A operand): row n, bytes 32 h2 .. +31 = logical chunks 2 h2 and 2 h2 + 1
    const int kf0 = n * D + (((2 * h2) ^ f8_swz(n)) * 16), kf1 = n * D + (((2 * h2 + 1) ^ f8_swz(n)) * 16);
    // V^T (A operand of O^T) through the transposing read: 16-lane group G = lane/16 covers
    // channels ct*32 + (G&1)*16 .. +15 and key half h2 = G>>1; lane L supplies row
    // key0 + L/4 (key0 = 16kb + 8t + 4h2) and channels cbase + 4(L%4) .. +3.
    const int G = lane >> 4, L = lane & 15;
    int voff[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int row = 4 * (G >> 1) + (L >> 2);
        const int c = ct * 4 + (G & 1) * 2 + ((L >> 1) & 1);
        voff[ct] = row * (kDV * 2) + v_phys(row, c) * 16 + (L & 1) * 8;
    }

    // ---- accumulators and softmax state (per lane = per query n, this lane's half of keys)
    f32x16 o1[4], o2[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) { o1[ct] = f32x16{}; o2[ct] = f32x16{}; }
    float m1 = -INFINITY, m2 = -INFINITY;
    // row sums in two partial chains per map (la: even key pairs, lb: odd), kept across tiles and
    // added once at the end
    float la1 = 0.f, lb1 = 0.f, la2 = 0.f, lb2 = 0.f;
    // score scale per map: softmax scale * log2(e), times the two fp8 dequantisation scales
    float c2a = a.scale_log2, c2b = a.scale_log2;
    if (F8) {
        const int64_t sh = (int64_t)b * a.heads + hout;
        c2a *= a.sq1[sh] * a.sk1[sh];
        c2b *= a.sq2[sh] * a.sk2[sh];
    }
    // rescale thresholds in raw score units, (m + 8) / c (c > 0); -inf until the first tile
    const float ic2a = 1.f / c2a, ic2b = 1.f / c2b;
    float th1 = -INFINITY, th2 = -INFINITY;
    bool started = false;   // a rescale has happened (wave-uniform)

    if (V2) {
        // this wave's 32 rows of Q_{2p+1} into its LDS region (rows of 16 chunks, swizzled like K;
        // rows past the end repeat the last row, whose outputs are not stored)
        const int qb0 = min(qw0, a.seq_q - 1);
        const bf16* qbase = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)qb0 * a.q2s[1] + (int64_t)hq2 * a.q2s[2];
#pragma unroll
        for (int i = 0; i < 32 * D * 2 / 1024; ++i) {
            const int c = lane + 64 * i;
            const int r = c / (D / 8), pc = c % (D / 8);
            const int qr = min(qw0 + r, a.seq_q - 1) - qb0;
            dma16(qbase, (uint32_t)(qr * a.q2s[1] + (pc ^ k_swz<D>(r)) * 8) * 2u,
                  smem_lds + C::Q2_OFF + wave_u * 32 * D * 2 + i * 1024);
        }
    }
    issue_tile(0, 0);

    // V1 lambda from its re-parameterisation (LAMF): the lambda kernel's arithmetic (lane-strided
    // fp32 dot products, the wave butterfly, expf), so the value is the one diffattn_lambda
    // writes; one block per head stores it. Placed after the first tile's DMA is issued, so the
    // vector loads overlap it.
    float lam_fused = 0.f;
    if (LAMF) {
        const int64_t base = (int64_t)hout * a.lam_dim;
        float d1 = 0.f, d2 = 0.f;
        for (int c = lane; c < a.lam_dim; c += 64) {
            d1 = fmaf(a.lq1[base + c], a.lk1[base + c], d1);
            d2 = fmaf(a.lq2[base + c], a.lk2[base + c], d2);
        }
        d1 = wave_sum(d1);
        d2 = wave_sum(d2);
        lam_fused = expf(d1) - expf(d2) + a.lambda_init;
        if (a.lam_out && b == 0 && qt == 0 && tid == 0) a.lam_out[hout] = lam_fused;
    }

    // one tile; the loop below is unrolled by the two stages so that each stage's LDS base is a
    // constant and folds into the operand reads' immediate offsets
    auto tile_step = [&](int kt, auto stage_c) __attribute__((always_inline)) {
        constexpr int stage = decltype(stage_c)::value;
        const int k0 = kt * kBN;
        const bool wave_needs = wave_active && (!CAUSAL || k0 <= wave_qlast + off);
        if (!wave_needs) return;
        const unsigned char* st = smem + stage * C::STAGE_BYTES;
        const unsigned char* Ks1 = st;
        const unsigned char* Ks2 = st + (C::NK - 1) * C::K_BYTES;
        const unsigned char* Vs = st + C::NK * C::K_BYTES;

        // S^T = K Q^T for both maps (fp32 accumulate)
        f32x16 s1 = f32x16{}, s2 = f32x16{};
        if (F8) {
            // one v_mfma_f32_32x32x64_f8f6f4 per map (OCP e4m3 operands, k = 64 = d)
            auto frag = [&](const unsigned char* t) __attribute__((always_inline)) {
                const u32x4 x0 = *(const u32x4*)(t + kf0), x1 = *(const u32x4*)(t + kf1);
                return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            };
            s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag(Ks1), fq1, s1, 0, 0, 0, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag(Ks2), fq2, s2, 0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8 ka = lds16(Ks1 + koff[kk]);
                s1 = mfma32x32x16(ka, bq1[kk], s1);
                if (V2) {
                    s2 = mfma32x32x16(ka, lds16(smem + C::Q2_OFF + wave_u * 32 * D * 2 + koff[kk]), s2);
                } else {
                    const bf16x8 kb2 = lds16(Ks2 + koff[kk]);
                    s2 = mfma32x32x16(kb2, bq2[kk], s2);
                }
            }
        }

        // mask keys past the end, and (causal) keys after the query's diagonal
        const bool need_mask = (k0 + kBN > a.seq_k) || (CAUSAL && k0 + kBN - 1 > qw0 + off);
        if (need_mask) {
            const int qlim = CAUSAL ? min(qrow + off, a.seq_k - 1) : a.seq_k - 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + (r >> 2) * 8 + h2 * 4 + (r & 3);
                if (key > qlim) { s1[r] = -INFINITY; s2[r] = -INFINITY; }
            }
        }

        // tile maxima (raw score units), shared by lanes n and n+32
        // a tree of 3-input maxima (depth 3, eight instructions per map): the maxima sit on the
        // path from the score MFMAs to the exponentials, so their depth counts, not just their number
        auto tile_max = [](const f32x16& x) __attribute__((always_inline)) {
            float t[6];
#pragma unroll
            for (int i = 0; i < 5; ++i) t[i] = fmax_nc(fmax_nc(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
            t[5] = x[15];
            return fmax_nc(fmax_nc(fmax_nc(t[0], t[1]), t[2]), fmax_nc(fmax_nc(t[3], t[4]), t[5]));
        };
        // compared in raw score units against the thresholds (m + 8) / c, which change only on a
        // rescale: no scaling of the maxima on the common path
        const float rx1 = max_halves(tile_max(s1)), rx2 = max_halves(tile_max(s2));
        const bool need = (rx1 > th1) || (rx2 > th2);
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mx1 = rx1 * c2a, mx2 = rx2 * c2b;
            const float mn1 = fmax_nc(m1, mx1), mn2 = fmax_nc(m2, mx2);
            const float al1 = fast_exp2(m1 - mn1), al2 = fast_exp2(m2 - mn2);
            m1 = mn1;
            m2 = mn2;
            th1 = (m1 + kRescaleThreshold) * ic2a;
            th2 = (m2 + kRescaleThreshold) * ic2b;
            la1 *= al1;
            lb1 *= al1;
            la2 *= al2;
            lb2 *= al2;
            // the wave's first rescale finds the accumulators still zero
            if (started) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) { o1[ct] *= al1; o2[ct] *= al2; }
            }
            started = true;
        }

        // Per half of the tile's keys (kb): unnormalised weights exp2(s*c - m) rounded to bf16
        // (the P^T operand), their row sums taken from the same bf16 values (v_dot2 with ones, so
        // numerator and normaliser use identical weights), then O^T += V^T P^T for both maps with
        // each V^T fragment feeding both. The MFMAs of the first half are interleaved with the
        // exponentials of the second half.
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
        bf16x8 p1[2], p2[2];
        auto softmax_half = [&](int kb) {
            bf16x2 q1p[4], q2p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kb * 8 + 2 * j;
                q1p[j] = bf16x2{(bf16)fast_exp2(fmaf(s1[r], c2a, -m1)), (bf16)fast_exp2(fmaf(s1[r + 1], c2a, -m1))};
                q2p[j] = bf16x2{(bf16)fast_exp2(fmaf(s2[r], c2b, -m2)), (bf16)fast_exp2(fmaf(s2[r + 1], c2b, -m2))};
                if (j & 1) {
                    lb1 = __builtin_amdgcn_fdot2_f32_bf16(q1p[j], ones, lb1, false);
                    lb2 = __builtin_amdgcn_fdot2_f32_bf16(q2p[j], ones, lb2, false);
                } else {
                    la1 = __builtin_amdgcn_fdot2_f32_bf16(q1p[j], ones, la1, false);
                    la2 = __builtin_amdgcn_fdot2_f32_bf16(q2p[j], ones, la2, false);
                }
            }
            p1[kb] = __builtin_shufflevector(__builtin_shufflevector(q1p[0], q1p[1], 0, 1, 2, 3),
                                             __builtin_shufflevector(q1p[2], q1p[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
            p2[kb] = __builtin_shufflevector(__builtin_shufflevector(q2p[0], q2p[1], 0, 1, 2, 3),
                                             __builtin_shufflevector(q2p[2], q2p[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 va[2][4];
        auto read_v = [&](int kb) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16* vp = (const bf16*)(Vs + voff[ct] + kb * 16 * (kDV * 2));
                const i16x4 lo = lds_read_tr16(vp);
                const i16x4 hi = lds_read_tr16(vp + 8 * kDV);
                va[kb][ct] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        auto pv = [&](int kb) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                o1[ct] = mfma32x32x16(va[kb][ct], p1[kb], o1[ct]);
                o2[ct] = mfma32x32x16(va[kb][ct], p2[kb], o2[ct]);
            }
        };
        read_v(0);
        softmax_half(0);
        constexpr bool kPrio = V2 ? DA_PRIO_V2 : DA_PRIO_V1;
        constexpr bool kSched = V2 ? DA_SCHED_V2 : DA_SCHED_V1;
        if (kPrio) __builtin_amdgcn_s_setprio(1);
        pv(0);
        softmax_half(1);
        read_v(1);
        pv(1);
        if (kPrio) __builtin_amdgcn_s_setprio(0);
        if (kSched) {
        // 8 V reads, the first half's softmax, then each first-half MFMA followed by a sixth of
        // the second half's softmax, the second half's V reads, and its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 48, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    };
    // V1: tiles in pairs, one block barrier per pair (half the barriers, and so half the waits for
    // the slowest wave): a ring of four stages holds the pair being computed and the next pair in
    // flight, 64 KB per block, two blocks per CU; unrolled by two pairs so every stage is a constant
    if (!V2 && 1 < nkt) issue_tile(1, 1);
    auto pair_step = [&](int kt, auto s0_c, auto s1_c, auto n0_c, auto n1_c) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): this thread's DMA of tiles kt, kt + 1 landed
        if ((kt + 1) * kBN > a.seq_k) zero_tail(kt, decltype(s0_c)::value);
        if (kt + 1 < nkt && (kt + 2) * kBN > a.seq_k) zero_tail(kt + 1, decltype(s1_c)::value);
        __syncthreads();                                    // both landed everywhere; the stages of the previous pair are free
        if (kt + 2 < nkt) issue_tile(kt + 2, decltype(n0_c)::value);
        if (kt + 3 < nkt) issue_tile(kt + 3, decltype(n1_c)::value);
        tile_step(kt, s0_c);
        if (kt + 1 < nkt) tile_step(kt + 1, s1_c);
    };
    if constexpr (!V2) {
        for (int kt = 0; kt < nkt; kt += 4) {
            pair_step(kt, StageC<0>{}, StageC<1>{}, StageC<2>{}, StageC<3>{});
            if (kt + 2 < nkt) pair_step(kt + 2, StageC<2>{}, StageC<3>{}, StageC<0>{}, StageC<1>{});
        }
    } else {
        // V2 (one block per CU, eight waves): two stages and a barrier per tile; pairing its tiles
        // measured no faster
        auto sync_step = [&](int kt, auto stage_c) __attribute__((always_inline)) {
            constexpr int stage = decltype(stage_c)::value;
            __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): this thread's DMA landed
            if ((kt + 1) * kBN > a.seq_k) zero_tail(kt, stage);
            __syncthreads();                                    // every DMA of tile kt landed; stage^1 free
            if (kt + 1 < nkt) issue_tile(kt + 1, stage ^ 1);    // prefetch overlaps this tile's compute
            tile_step(kt, stage_c);
        };
        for (int kt = 0; kt < nkt; kt += 2) {
            sync_step(kt, StageC<0>{});
            if (kt + 1 < nkt) sync_step(kt + 1, StageC<1>{});
        }
    }

    if (!wave_active) return;

    // ---- epilogue: O = O1/l1 - lambda O2/l2 (+ RMSNorm * w * (1 - lambda_init))
    const float l1 = sum_halves(la1 + lb1);
    const float l2 = sum_halves(la2 + lb2);
    float lam;
    if (V2) {
        lam = (qrow < a.seq_q) ? a.lam[b * a.lams[0] + (int64_t)qrow * a.lams[1] + (int64_t)hout * a.lams[2]] : 0.f;
        if (a.lam_sigmoid) lam = sigmoid_f32(lam);
    } else {
        lam = LAMF ? lam_fused : a.lam[hout];
    }
    const float r1 = 1.f / l1;
    const float r2 = lam / l2;
    if (a.lse && qrow < a.seq_q) {
        // training outputs for the backward pass: each map's log-sum-exp in base 2 (in the units
        // of the scaled scores, so a weight is exp2(c s - lse)) and its normalised output A_k V
        const int64_t row = ((int64_t)b * a.heads + hout) * a.seq_q + qrow;
        if (h2 == 0) {
            a.lse[2 * row] = m1 + log2f(l1);
            a.lse[2 * row + 1] = m2 + log2f(l2);
        }
        const float i2 = 1.f / l2;
        float* mp = a.maps + row_major_maps(a, b, qrow, hout);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x1, x2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x1[j] = o1[ct][g * 4 + j] * r1;
                    x2[j] = o2[ct][g * 4 + j] * i2;
                }
                const int c = ct * 32 + g * 8 + h2 * 4;
                *(f32x4*)(mp + c) = x1;
                *(f32x4*)(mp + kDV + c) = x2;
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // both products rounded before the difference: identical maps with lambda = 1 cancel
            // exactly (no fused multiply-add here)
#pragma clang fp contract(off)
            const float x = o1[ct][r] * r1 - o2[ct][r] * r2;
            o1[ct][r] = x;
            ss = fmaf(x, x, ss);
        }
    }
    if (EPI) {
        ss = sum_halves(ss);
        const float inv = (1.f / sqrtf(ss * (1.f / kDV) + a.eps)) * (1.f - a.lambda_init);
        // the weight test is made once, not per channel
        if (a.norm_w) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = ct * 32 + (r >> 2) * 8 + h2 * 4 + (r & 3);
                    o1[ct][r] *= inv * a.norm_w[c];
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) o1[ct] *= inv;
        }
    }
    if (qrow < a.seq_q) {
        bf16* op = (bf16*)a.out + b * a.os[0] + (int64_t)qrow * a.os[1] + (int64_t)hout * a.os[2];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = (bf16)o1[ct][g * 4 + j];
                *(bf16x4*)(op + ct * 32 + g * 8 + h2 * 4) = pk;
            }
        }
    }
}

template <int D, bool V2, bool F8 = false>
hipError_t launch_fwd(const MfmaFwdArgs& a, hipStream_t stream) {
    using C = Cfg<D, V2, F8>;
    const int pairs_per_block = V2 ? a.kv_group / 2 : 1;
    const int BM = 32 * (C::NW / pairs_per_block);
    const int n_units = V2 ? a.batch * (a.heads * 2 / a.kv_group) : a.batch * a.heads;
    const int nqt = (a.seq_q + BM - 1) / BM;
    const dim3 grid((unsigned)(nqt * n_units));
    const size_t smem = 0;   // the kernel's LDS is static
    if (!V2 && !F8 && a.lq1) {   // lambda from its vectors inside the kernel
        if (a.causal) {
            if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, true, F8, true>), grid, dim3(C::NT), smem, stream, a);
            else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, false, F8, true>), grid, dim3(C::NT), smem, stream, a);
        } else {
            if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, true, F8, true>), grid, dim3(C::NT), smem, stream, a);
            else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, false, F8, true>), grid, dim3(C::NT), smem, stream, a);
        }
        return hipGetLastError();
    }
    if (a.causal) {
        if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, true, F8>), grid, dim3(C::NT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, false, F8>), grid, dim3(C::NT), smem, stream, a);
    } else {
        if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, true, F8>), grid, dim3(C::NT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, false, F8>), grid, dim3(C::NT), smem, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

}  // namespace diffattn
