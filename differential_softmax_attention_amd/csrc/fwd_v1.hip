// DIFF V1 forward on bf16 MFMA (gfx950): d = 64 per map, dv = 128, optional RMSNorm epilogue.
//
// Computes, per query row, O = softmax(s Q1 K1^T) V - lambda softmax(s Q2 K2^T) V, which equals
// (A1 - lambda A2) V exactly ("Differential Transformer: softmax can't say zero, so it subtracts",
// section "What it costs": a fused kernel computes A1 V and A2 V because the maps are never
// materialised), then O / rms(O) * w * (1 - lambda_init) ("Noise-Canceling Attention by
// Subtraction", sections "The mechanism" and "Making lambda learnable and stable").
//
// Design (one pass over K/V, both maps at once):
//  - A block of 4 waves owns 128 query rows of one head; each wave owns 32 rows. K1, K2 and V
//    tiles of 32 keys are staged through a 3-deep LDS ring by global_load_lds, so every tile is
//    read from memory once per block and V once for both maps.
//  - Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane (n, h)
//    holds 16 keys of query n, so row sums are per-lane values. The output is accumulated
//    transposed, O^T += V^T P^T, with V^T read by the transposing LDS read (ds_read_b64_tr_b16).
//  - Software pipeline inside each wave: while the exponentials of tile t run on the VALU, the
//    MFMA unit works on P(t-1) V(t-1). This is why the ring is 3 deep: the V of tile t-1 is still
//    read while tile t is current and tile t+1 arrives. Two waves share each SIMD, so each has
//    256 registers; the pipeline fits in them with one score tile and two weight tiles live.
//  - Softmax in base 2 with Q pre-multiplied by scale * log2(e). A wave whose first-tile row
//    maxima lie within 2^+-60 runs unshifted: a weight is exp2(S), one exponential per score, no
//    running maximum. Should a tile's weights leave a safe range (a lane's 16 weights summing
//    above 2^64, or to a non-finite value), the wave switches to shifted mode, where scores are
//    reduced by a per-row shift that only rises; O and the sums are rescaled when it moves.
//    Numerator and normaliser always use the same weights, so the result is the softmax.
//  - Epilogue in registers: O1/l1 - lambda O2/l2, then RMSNorm over the 128 channels and the
//    (1 - lambda_init) multiply, stored as bf16.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tile.hpp"

namespace diffattn {

namespace {

constexpr int kBN = 32;                 // keys per tile
constexpr int kD = 64;                  // query / key width per map
constexpr int kDV = 128;                // value width
constexpr int kNW = 4;                  // waves per block
constexpr int kNT = kNW * 64;
constexpr int kBM = 32 * kNW;           // query rows per block
constexpr int kKBytes = kBN * kD * 2;
constexpr int kVBytes = kBN * kDV * 2;
constexpr int kStageBytes = 2 * kKBytes + kVBytes;
constexpr int kStages = 3;
constexpr int kVLoads = kBN * (kDV / 8) / kNT;   // V DMA loads per thread per tile
static_assert(kBN * (kD / 8) == kNT && kVLoads == 2, "tile / block shape");

constexpr float kMaxSum = 18446744073709551616.0f;  // 2^64: bound on a lane's 16 weights, unshifted
constexpr float kMaxSumShifted = 32768.0f;          // 2^15: the same bound in shifted mode
constexpr float kMinSum = 8.673617379884035e-19f;   // 2^-60: a row below this has no weight yet
constexpr float kUnshiftedRange = 60.0f;            // first-tile row maxima within +-60 (base 2)

// raised wave priority while issuing the P V MFMAs, and explicit interleave of those MFMAs
// with the next tile's softmax (VALU instructions per MFMA; 0 leaves it to the compiler)
#ifndef DA_V1_PRIO
#define DA_V1_PRIO 1
#endif
#ifndef DA_V1_SCHED
#define DA_V1_SCHED 0
#endif

template <bool CAUSAL, bool EPI>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_v1_kernel(MfmaFwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    // The wave index stays a per-lane value for control flow: treating it as uniform lets the
    // compiler restructure the loop in ways that spill registers. Addresses take a copy in SGPRs.
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;   // query column within the wave's 32 rows
    const int h2 = lane >> 5;  // which half of the MFMA k-dimension this lane feeds

    // ---- block -> (query tile, head, batch); heavy causal tiles first, and the tiles of one
    //      head kept on one XCD (blocks are dealt round-robin over 8 XCDs).
    const int n_units = a.batch * a.heads;
    const int nqt = (a.seq_q + kBM - 1) / kBM;
    int unit, qt;
    {
        const int bid = blockIdx.x;
        if ((n_units & 7) == 0) {
            const int per = n_units >> 3;
            const int slot = bid >> 3;
            unit = (bid & 7) * per + slot % per;
            qt = slot / per;
        } else {
            unit = bid % n_units;
            qt = bid / n_units;
        }
        if (CAUSAL) qt = nqt - 1 - qt;
    }
    const int b = unit / a.heads;
    const int h = unit % a.heads;
    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * 32;       // first query row of this wave
    const int qrow = qw0 + n;
    const int off = a.seq_k - a.seq_q;    // causal alignment to the last key

    // ---- Q fragments (B operand of S^T = K Q^T): lane (n, h2) holds c*q[n][16kk + 8h2 .. +7],
    //      pre-multiplied by c = scale * log2(e) (rounded to bf16), so scores come out of the
    //      MFMA in base-2 units.
    constexpr int NKK = kD / 16;
    bf16x8 bq1[NKK], bq2[NKK];
    {
        const bool ok = qrow < a.seq_q;
        const int qr = ok ? qrow : 0;
        const bf16* q1p = (const bf16*)a.q1 + b * a.q1s[0] + (int64_t)qr * a.q1s[1] + (int64_t)h * a.q1s[2] + 8 * h2;
        const bf16* q2p = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)qr * a.q2s[1] + (int64_t)h * a.q2s[2] + 8 * h2;
        const float c = a.scale_log2;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const bf16x8 z = {};
            const bf16x8 x1 = ok ? ld_global_bf16x8(q1p + 16 * kk) : z;
            const bf16x8 x2 = ok ? ld_global_bf16x8(q2p + 16 * kk) : z;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bq1[kk][j] = (bf16)((float)x1[j] * c);
                bq2[kk][j] = (bf16)((float)x2[j] * c);
            }
        }
    }

    // ---- key range of the block and of this wave
    int nkt = (a.seq_k + kBN - 1) / kBN;
    if (CAUSAL) nkt = min(nkt, (min(q0 + kBM, a.seq_q) - 1 + off) / kBN + 1);
    int wave_nkt = 0;   // tiles this wave reads (a prefix of the block's tiles)
    if (qw0 < a.seq_q) wave_nkt = CAUSAL ? min(nkt, (min(qw0 + 31, a.seq_q - 1) + off) / kBN + 1) : nkt;

    // ---- tile DMA: thread tid fills K slot tid (of K1 and of K2) and V slots tid, tid + 256.
    //      Slot s of K holds row s / 8, logical chunk (s % 8) ^ k_swz(row); slot s of V holds
    //      row s / 16, logical chunk v_logical(row, s % 16). Rows of a partial last tile are
    //      clamped to the last key.
    const bf16* kbase1 = (const bf16*)a.k1 + b * a.k1s[0] + (int64_t)h * a.k1s[2];
    const bf16* kbase2 = (const bf16*)a.k2 + b * a.k2s[0] + (int64_t)h * a.k2s[2];
    const bf16* vbase = (const bf16*)a.v + b * a.vs[0] + (int64_t)h * a.vs[2];
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(lds_u8_t*)smem + __builtin_amdgcn_readfirstlane(wave) * 64 * 16;

    // per-thread byte offsets of its chunks within a full tile; a partial last tile recomputes
    // them with rows clamped to the last key
    const int k_row = tid >> 3;
    const int k_col = (tid & 7) ^ k_swz<kD>(k_row);
    const int v_row0 = tid >> 4, v_row1 = v_row0 + 16;
    const int v_col0 = v_logical(v_row0, tid & 15), v_col1 = v_logical(v_row1, tid & 15);
    const uint32_t dk1 = (uint32_t)(k_row * a.k1s[1] + k_col * 8) * 2u;
    const uint32_t dk2 = (uint32_t)(k_row * a.k2s[1] + k_col * 8) * 2u;
    const uint32_t dv0 = (uint32_t)(v_row0 * a.vs[1] + v_col0 * 8) * 2u;
    const uint32_t dv1 = (uint32_t)(v_row1 * a.vs[1] + v_col1 * 8) * 2u;
    const int full_tiles = a.seq_k / kBN;

    auto issue_tile = [&](int kt, int stage) __attribute__((always_inline)) {
        const uint32_t st = lds_wave + stage * kStageBytes;
        const bf16* k1b = kbase1 + (int64_t)kt * kBN * a.k1s[1];
        const bf16* k2b = kbase2 + (int64_t)kt * kBN * a.k2s[1];
        const bf16* vb = vbase + (int64_t)kt * kBN * a.vs[1];
        if (kt < full_tiles) {
            dma16(k1b, dk1, st);
            dma16(k2b, dk2, st + kKBytes);
            dma16(vb, dv0, st + 2 * kKBytes);
            dma16(vb, dv1, st + 2 * kKBytes + kNT * 16);
        } else {
            const int last = a.seq_k - 1 - kt * kBN;   // last valid row within this tile
            const int kr = min(k_row, last);
            dma16(k1b, (uint32_t)(kr * a.k1s[1] + k_col * 8) * 2u, st);
            dma16(k2b, (uint32_t)(kr * a.k2s[1] + k_col * 8) * 2u, st + kKBytes);
            dma16(vb, (uint32_t)(min(v_row0, last) * a.vs[1] + v_col0 * 8) * 2u, st + 2 * kKBytes);
            dma16(vb, (uint32_t)(min(v_row1, last) * a.vs[1] + v_col1 * 8) * 2u, st + 2 * kKBytes + kNT * 16);
        }
    };
    // rows past the last key were fetched from a clamped address; zero them once the DMA landed
    // (only the last tile can have such rows)
    auto zero_tail = [&](int kt, int stage) __attribute__((always_inline)) {
        unsigned char* st = smem + stage * kStageBytes;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (kt * kBN + (tid >> 3) >= a.seq_k) {
            *(u32x4*)(st + tid * 16) = z;
            *(u32x4*)(st + kKBytes + tid * 16) = z;
        }
#pragma unroll
        for (int j = 0; j < kVLoads; ++j) {
            const int s = tid + j * kNT;
            if (kt * kBN + (s >> 4) >= a.seq_k) *(u32x4*)(st + 2 * kKBytes + s * 16) = z;
        }
    };

    // ---- per-lane LDS offsets of the MFMA operands
    // K (A operand of S^T): row n, logical chunk 2kk + h2, physical chunk (2kk + h2) ^ k_swz(n);
    // 2kk only touches chunk bits the base never sets, so block kk is at koff0 ^ (kk << 5).
    const int koff0 = n * (kD * 2) + ((h2 ^ k_swz<kD>(n)) * 16);
    // V^T (A operand of O^T) through the transposing read: 16-lane group G = lane/16 covers
    // channels ct*32 + (G&1)*16 .. +15 and key half h2 = G>>1; lane L supplies row
    // key0 + L/4 (key0 = 16kb + 8t + 4h2) and channels cbase + 4(L%4) .. +3. The channel tile ct
    // only flips chunk bits 2-3, so tile ct is at voff0 ^ (ct << 6).
    int voff0;
    {
        const int G = lane >> 4, L = lane & 15;
        const int row = 4 * (G >> 1) + (L >> 2);
        const int c = (G & 1) * 2 + ((L >> 1) & 1);
        voff0 = row * (kDV * 2) + v_phys(row, c) * 16 + (L & 1) * 8;
    }

    // ---- accumulators and softmax state (per lane = per query n, this lane's half of keys)
    f32x16 o1[4], o2[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) { o1[ct] = f32x16{}; o2[ct] = f32x16{}; }
    float m1 = 0.f, m2 = 0.f, l1 = 0.f, l2 = 0.f;   // per-map shift and running sum
    bool shifted = false;

    // S^T = K (cQ)^T for both maps (fp32 accumulate), in base-2 units
    auto qk = [&](const unsigned char* st, f32x16& s1, f32x16& s2) __attribute__((always_inline)) {
        s1 = f32x16{};
        s2 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int koff = koff0 ^ (kk << 5);
            s1 = mfma32x32x16(lds16(st + koff), bq1[kk], s1);
            s2 = mfma32x32x16(lds16(st + kKBytes + koff), bq2[kk], s2);
        }
    };
    // keys past the end, and (causal) keys after the query's diagonal, get -inf in both maps
    auto mask = [&](int k0, f32x16& s1, f32x16& s2) __attribute__((always_inline)) {
        const int qlim = CAUSAL ? min(qrow + off, a.seq_k - 1) : a.seq_k - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + (r >> 2) * 8 + h2 * 4 + (r & 3);
            if (key > qlim) { s1[r] = -INFINITY; s2[r] = -INFINITY; }
        }
    };
    // O^T += V^T P^T for both maps; each V^T fragment (transposing LDS read) feeds both
    auto pv = [&](const unsigned char* Vs, const bf16x8 (&p1)[2], const bf16x8 (&p2)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16* vp = (const bf16*)(Vs + (voff0 ^ (ct << 6)) + kb * 16 * (kDV * 2));
                const i16x4 lo = lds_read_tr16(vp);
                const i16x4 hi = lds_read_tr16(vp + 8 * kDV);
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o1[ct] = mfma32x32x16(va, p1[kb], o1[ct]);
                o2[ct] = mfma32x32x16(va, p2[kb], o2[ct]);
            }
        }
    };
    // Shifted mode: move the shift of both maps by this tile's row maxima (floored at 0 once the
    // row has weight, so the shift only rises and O and l only shrink); O and l are rescaled by
    // 2^-(shift change) and the tile's scores reduced by the same amount. Lanes n and n+32 share
    // query n and take identical decisions.
    auto move_shift = [&](f32x16& s1, f32x16& s2) __attribute__((always_inline)) {
        float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) { mx1 = fmax_nc(mx1, s1[r]); mx2 = fmax_nc(mx2, s2[r]); }
        mx1 = max_halves(mx1);
        mx2 = max_halves(mx2);
        if (!(sum_halves(l1) < kMinSum)) mx1 = fmax_nc(mx1, 0.f);
        if (!(sum_halves(l2) < kMinSum)) mx2 = fmax_nc(mx2, 0.f);
        const float al1 = fast_exp2(-mx1), al2 = fast_exp2(-mx2);
        l1 *= al1;
        l2 *= al2;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) { o1[ct] *= al1; o2[ct] *= al2; }
#pragma unroll
        for (int r = 0; r < 16; ++r) { s1[r] -= mx1; s2[r] -= mx2; }
        m1 += mx1;
        m2 += mx2;
    };
    // Weights exp2(S) rounded to bf16 (the P^T operands, one per half of the tile's keys), with
    // this lane's sums taken from the same bf16 values (v_dot2 with ones), so numerator and
    // normaliser use identical weights.
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    auto weights = [&](const f32x16& s1, const f32x16& s2, bf16x8 (&p1)[2], bf16x8 (&p2)[2], float& ls1,
                       float& ls2) __attribute__((always_inline)) {
        float a1 = 0.f, b1 = 0.f, a2 = 0.f, b2 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x2 q1p[4], q2p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kb * 8 + 2 * j;
                q1p[j] = bf16x2{(bf16)fast_exp2(s1[r]), (bf16)fast_exp2(s1[r + 1])};
                q2p[j] = bf16x2{(bf16)fast_exp2(s2[r]), (bf16)fast_exp2(s2[r + 1])};
                if (j & 1) {
                    b1 = __builtin_amdgcn_fdot2_f32_bf16(q1p[j], ones, b1, false);
                    b2 = __builtin_amdgcn_fdot2_f32_bf16(q2p[j], ones, b2, false);
                } else {
                    a1 = __builtin_amdgcn_fdot2_f32_bf16(q1p[j], ones, a1, false);
                    a2 = __builtin_amdgcn_fdot2_f32_bf16(q2p[j], ones, a2, false);
                }
            }
            p1[kb] = __builtin_shufflevector(__builtin_shufflevector(q1p[0], q1p[1], 0, 1, 2, 3),
                                             __builtin_shufflevector(q1p[2], q1p[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
            p2[kb] = __builtin_shufflevector(__builtin_shufflevector(q2p[0], q2p[1], 0, 1, 2, 3),
                                             __builtin_shufflevector(q2p[2], q2p[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        }
        ls1 = a1 + b1;
        ls2 = a2 + b2;
    };
    // A lane's sixteen weights must sum to at most 2^64 unshifted (2^15 shifted) and to a finite
    // value, so no weight, sum or accumulator can overflow; if any lane fails, the wave enters
    // shifted mode and redoes the tile's weights. Ordinary scores never trigger this.
    auto check = [&](f32x16& s1, f32x16& s2, bf16x8 (&p1)[2], bf16x8 (&p2)[2], float& ls1, float& ls2)
        __attribute__((always_inline)) {
        const float lim = __builtin_amdgcn_readfirstlane(shifted) ? kMaxSumShifted : kMaxSum;
        const bool bad = !(ls1 <= lim) || !(ls2 <= lim);
        if (__builtin_amdgcn_ballot_w64(bad)) {
            shifted = true;
            move_shift(s1, s2);
            weights(s1, s2, p1, p2, ls1, ls2);
        }
        l1 += ls1;
        l2 += ls2;
    };

    // ---- tile loop. Tile kt sits in ring stage kt % 3. At the top of step kt each thread waits
    //      for its own DMA of tile kt, the barrier publishes the tile and guarantees that every
    //      wave has finished step kt-1 (which read V of tile kt-2), and tile kt+1 is then fetched
    //      into the stage of tile kt-2. Step kt computes S(kt) and P(kt) and accumulates
    //      P(kt-1) V(kt-1); a wave's last P V runs one step after its last tile (or after the loop).
    auto top = [&](int kt, int stage) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt[0]);
        if ((kt + 1) * kBN > a.seq_k) zero_tail(kt, stage);
        __syncthreads();
        if (kt + 1 < nkt) issue_tile(kt + 1, stage == kStages - 1 ? 0 : stage + 1);
    };

    issue_tile(0, 0);
    bf16x8 pp1[2], pp2[2];   // weights of the previous tile
    int prev = 0;            // its stage
    top(0, 0);
    if (wave_nkt > 0) {
        f32x16 s1, s2;
        qk(smem, s1, s2);
        if (kBN > a.seq_k || (CAUSAL && kBN - 1 > qw0 + off)) mask(0, s1, s2);
        // The first tile's row maxima decide the mode (key 0 is visible, so they are finite and no
        // later tile can underflow a row to zero weight).
        {
            float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) { mx1 = fmax_nc(mx1, s1[r]); mx2 = fmax_nc(mx2, s2[r]); }
            const bool far = !(fabsf(mx1) <= kUnshiftedRange) || !(fabsf(mx2) <= kUnshiftedRange);
            if (__builtin_amdgcn_ballot_w64(far)) {
                move_shift(s1, s2);
                shifted = true;
            }
        }
        float ls1, ls2;
        weights(s1, s2, pp1, pp2, ls1, ls2);
        check(s1, s2, pp1, pp2, ls1, ls2);
    }
    int stage = 0;
    for (int kt = 1; kt < nkt; ++kt) {
        stage = stage == kStages - 1 ? 0 : stage + 1;
        top(kt, stage);
        if (kt < wave_nkt) {
            const int k0 = kt * kBN;
            const unsigned char* st = smem + stage * kStageBytes;
            f32x16 s1, s2;
            qk(st, s1, s2);
            const bool need_mask = (k0 + kBN > a.seq_k) || (CAUSAL && k0 + kBN - 1 > qw0 + off);
            if (need_mask || shifted) {
                if (need_mask) mask(k0, s1, s2);
                if (shifted) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) { s1[r] -= m1; s2[r] -= m2; }
                }
            }
            if (DA_V1_PRIO) __builtin_amdgcn_s_setprio(1);
            pv(smem + prev * kStageBytes + 2 * kKBytes, pp1, pp2);
            if (DA_V1_PRIO) __builtin_amdgcn_s_setprio(0);
            bf16x8 p1[2], p2[2];
            float ls1, ls2;
            weights(s1, s2, p1, p2, ls1, ls2);
            if (DA_V1_SCHED) {
                // the first two V^T fragments, then per MFMA one V^T read (while any are left) and
                // a few VALU instructions of this tile's weights
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, DA_V1_SCHED, 0);
                }
            }
            check(s1, s2, p1, p2, ls1, ls2);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) { pp1[kb] = p1[kb]; pp2[kb] = p2[kb]; }
            prev = stage;
        } else if (kt == wave_nkt) {
            pv(smem + prev * kStageBytes + 2 * kKBytes, pp1, pp2);
        }
    }
    if (wave_nkt == 0) return;
    if (wave_nkt == nkt) pv(smem + prev * kStageBytes + 2 * kKBytes, pp1, pp2);

    // ---- epilogue: O = O1/l1 - lambda O2/l2 (+ RMSNorm * w * (1 - lambda_init))
    l1 = sum_halves(l1);
    l2 = sum_halves(l2);
    const float lam = a.lam[h];
    const float r1 = 1.f / l1;
    const float r2 = lam / l2;
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
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = ct * 32 + (r >> 2) * 8 + h2 * 4 + (r & 3);
                const float w = a.norm_w ? a.norm_w[c] : 1.f;
                o1[ct][r] *= inv * w;
            }
        }
    }
    if (qrow < a.seq_q) {
        bf16* op = (bf16*)a.out + b * a.os[0] + (int64_t)qrow * a.os[1] + (int64_t)h * a.os[2];
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

}  // namespace

hipError_t launch_v1_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream) {
    const int nqt = (a.seq_q + kBM - 1) / kBM;
    const dim3 grid((unsigned)(nqt * a.batch * a.heads));
    const size_t smem = (size_t)kStages * kStageBytes;
    if (a.causal) {
        if (a.epi) hipLaunchKernelGGL((fwd_v1_kernel<true, true>), grid, dim3(kNT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_v1_kernel<true, false>), grid, dim3(kNT), smem, stream, a);
    } else {
        if (a.epi) hipLaunchKernelGGL((fwd_v1_kernel<false, true>), grid, dim3(kNT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_v1_kernel<false, false>), grid, dim3(kNT), smem, stream, a);
    }
    return hipGetLastError();
}

}  // namespace diffattn
