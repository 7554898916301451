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
//    Each wave owns 32 query rows of one pair. K/V tiles of 32 keys are staged through LDS,
//    double buffered, so every tile is read from memory once per block and V once for both maps.
//  - Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane (n, h)
//    then holds 16 keys of query n, so the running max and sum of each map are per-lane values
//    (one exchange between lanes n and n+32 per tile).
//  - The output is accumulated transposed, O^T += V^T P^T: P^T comes straight from the score
//    registers (rounded to bf16), V^T is read from the row-major V tile with the gfx950
//    transposing LDS read (ds_read_b64_tr_b16), so V is never transposed in registers.
//  - Online softmax per map in base 2 (scale * log2 e folded into one FMA). The running maximum
//    is only raised when a tile's maximum exceeds it by more than 8 (so unnormalised weights stay
//    below 2^8); the final normalisation uses the same maximum, so the result is unchanged.
//  - Epilogue in registers: O1/l1 - lambda O2/l2, then (V1) RMSNorm over the 128 channels and the
//    (1 - lambda_init) multiply, stored as bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

constexpr int kBN = 32;          // keys per tile
constexpr int kDV = 128;         // value width
constexpr int kVP = kDV + 16;    // LDS pitch of a V row (elements)
constexpr float kRescaleThreshold = 8.0f;

template <int D, bool V2>
struct Cfg {
    static constexpr int NW = V2 ? 8 : 4;              // waves per block
    static constexpr int NT = NW * 64;
    static constexpr int KP = D + 8;                    // LDS pitch of a K row (elements)
    static constexpr int NK = V2 ? 1 : 2;               // K tiles per stage (V2 shares K)
    static constexpr int K_ELEMS = kBN * KP;
    static constexpr int V_ELEMS = kBN * kVP;
    static constexpr int STAGE = NK * K_ELEMS + V_ELEMS;
    static constexpr int KCH = kBN * D / 8;             // 16-byte chunks per K tile
    static constexpr int VCH = kBN * kDV / 8;
    static constexpr int TOT = NK * KCH + VCH;
    static_assert(TOT % NT == 0, "tile chunks must divide evenly");
    static constexpr int PER = TOT / NT;
};

__device__ __forceinline__ u32x4 ld_global16(const bf16* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st_lds16(bf16* p, u32x4 x) { *(u32x4*)p = x; }
__device__ __forceinline__ bf16x8 ld_lds16(const bf16* p) { return *(const bf16x8*)p; }

template <int D, bool V2, bool CAUSAL, bool EPI>
__global__ __launch_bounds__(V2 ? 512 : 256) void fwd_mfma_kernel(MfmaFwdArgs a) {
    using C = Cfg<D, V2>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    bf16* smem = (bf16*)smem_raw;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
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
    const int n_groups = V2 ? (a.heads * 2 / a.kv_group) : a.heads;
    const int b = unit / n_groups;
    const int grp = unit % n_groups;      // V1: head; V2: KV head
    const int pair_in_grp = wave % pairs_per_block;
    const int qsub = wave / pairs_per_block;
    const int q0 = qt * BM;
    const int qw0 = q0 + qsub * 32;       // first query row of this wave
    const int qrow = qw0 + n;
    const int off = a.seq_k - a.seq_q;    // causal alignment to the last key

    // heads read by this wave
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
    {
        const bf16* q1p = (const bf16*)a.q1 + b * a.q1s[0] + (int64_t)qrow * a.q1s[1] + (int64_t)hq1 * a.q1s[2] + 8 * h2;
        const bf16* q2p = (const bf16*)a.q2 + b * a.q2s[0] + (int64_t)qrow * a.q2s[1] + (int64_t)hq2 * a.q2s[2] + 8 * h2;
        const bool ok = qrow < a.seq_q;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            bf16x8 z = {};
            bq1[kk] = ok ? ld_lds16(q1p + 16 * kk) : z;   // (plain 16-byte global loads)
            bq2[kk] = ok ? ld_lds16(q2p + 16 * kk) : z;
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

    // ---- cooperative tile loader: chunk c of a stage = (tensor, row, 16-byte column)
    const bf16* kbase1 = (const bf16*)a.k1 + b * a.k1s[0] + (int64_t)kvh * a.k1s[2];
    const bf16* kbase2 = (const bf16*)a.k2 + b * a.k2s[0] + (int64_t)kvh * a.k2s[2];
    const bf16* vbase = (const bf16*)a.v + b * a.vs[0] + (int64_t)kvh * a.vs[2];
    u32x4 stage_regs[C::PER];

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < C::PER; ++i) {
            const int c = tid + i * C::NT;
            const bf16* src;
            int row;
            if (c < C::NK * C::KCH) {
                const int cc = c % C::KCH;
                row = cc / (D / 8);
                const int col = (cc % (D / 8)) * 8;
                const bf16* kb = (c < C::KCH) ? kbase1 : kbase2;
                const int64_t rs = (c < C::KCH) ? a.k1s[1] : a.k2s[1];
                src = kb + (int64_t)(kt * kBN + row) * rs + col;
            } else {
                const int cc = c - C::NK * C::KCH;
                row = cc / (kDV / 8);
                const int col = (cc % (kDV / 8)) * 8;
                src = vbase + (int64_t)(kt * kBN + row) * a.vs[1] + col;
            }
            u32x4 z = {0u, 0u, 0u, 0u};
            stage_regs[i] = (kt * kBN + row < a.seq_k) ? ld_global16(src) : z;
        }
    };
    auto store_tile = [&](int stage) {
        bf16* st = smem + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::PER; ++i) {
            const int c = tid + i * C::NT;
            bf16* dst;
            if (c < C::NK * C::KCH) {
                const int which = c / C::KCH;
                const int cc = c % C::KCH;
                dst = st + which * C::K_ELEMS + (cc / (D / 8)) * C::KP + (cc % (D / 8)) * 8;
            } else {
                const int cc = c - C::NK * C::KCH;
                dst = st + C::NK * C::K_ELEMS + (cc / (kDV / 8)) * kVP + (cc % (kDV / 8)) * 8;
            }
            st_lds16(dst, stage_regs[i]);
        }
    };

    // ---- accumulators and softmax state (per lane = per query n, this lane's half of keys)
    f32x16 o1[4], o2[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) { o1[ct] = f32x16{}; o2[ct] = f32x16{}; }
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    const float c2 = a.scale_log2;
    const int xaddr = (lane ^ 32) << 2;

    // V^T operand addressing for the transposing read (see the layout note above):
    // 16-lane group G = lane/16 covers channels ct*32 + (G&1)*16 .. +15 and key half h2 = G>>1;
    // lane L in the group supplies row key0 + L/4, channels cbase + 4(L%4).
    const int G = lane >> 4, L = lane & 15;
    const int v_lane_off = ((G >> 1) * 4 + (L >> 2)) * kVP + (G & 1) * 16 + 4 * (L & 3);

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const bool has_next = kt + 1 < nkt;
        if (has_next) load_tile(kt + 1);

        const int k0 = kt * kBN;
        const bool wave_needs = wave_active && (!CAUSAL || k0 <= wave_qlast + off);
        if (wave_needs) {
            const bf16* st = smem + (kt & 1) * C::STAGE;
            const bf16* Ks1 = st;
            const bf16* Ks2 = st + (C::NK - 1) * C::K_ELEMS;
            const bf16* Vs = st + C::NK * C::K_ELEMS;

            // S^T = K Q^T for both maps (fp32 accumulate)
            f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8 ka = ld_lds16(Ks1 + n * C::KP + 16 * kk + 8 * h2);
                s1 = mfma32x32x16(ka, bq1[kk], s1);
                if (V2) {
                    s2 = mfma32x32x16(ka, bq2[kk], s2);
                } else {
                    const bf16x8 kb2 = ld_lds16(Ks2 + n * C::KP + 16 * kk + 8 * h2);
                    s2 = mfma32x32x16(kb2, bq2[kk], s2);
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
            float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) { mx1 = fmaxf(mx1, s1[r]); mx2 = fmaxf(mx2, s2[r]); }
            mx1 = fmaxf(mx1, lane_xor(mx1, xaddr)) * c2;
            mx2 = fmaxf(mx2, lane_xor(mx2, xaddr)) * c2;
            const bool need = (mx1 > m1 + kRescaleThreshold) || (mx2 > m2 + kRescaleThreshold);
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn1 = fmaxf(m1, mx1), mn2 = fmaxf(m2, mx2);
                const float al1 = fast_exp2(m1 - mn1), al2 = fast_exp2(m2 - mn2);
                m1 = mn1;
                m2 = mn2;
                l1 *= al1;
                l2 *= al2;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) { o1[ct] *= al1; o2[ct] *= al2; }
            }

            // unnormalised weights, their sums, and the bf16 P^T operands
            bf16x8 p1[2], p2[2];
            float ls1 = 0.f, ls2 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e1 = fast_exp2(fmaf(s1[r], c2, -m1));
                const float e2 = fast_exp2(fmaf(s2[r], c2, -m2));
                ls1 += e1;
                ls2 += e2;
                p1[r >> 3][r & 7] = (bf16)e1;
                p2[r >> 3][r & 7] = (bf16)e2;
            }
            l1 += ls1;
            l2 += ls2;

            // O^T += V^T P^T for both maps; each V^T fragment feeds both
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16* vp = Vs + (kb * 16) * kVP + ct * 32 + v_lane_off;
                    const i16x4 lo = lds_read_tr16(vp);
                    const i16x4 hi = lds_read_tr16(vp + 8 * kVP);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o1[ct] = mfma32x32x16(va, p1[kb], o1[ct]);
                    o2[ct] = mfma32x32x16(va, p2[kb], o2[ct]);
                }
            }
        }

        if (has_next) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    if (!wave_active) return;

    // ---- epilogue: O = O1/l1 - lambda O2/l2 (+ RMSNorm * w * (1 - lambda_init))
    l1 += lane_xor(l1, xaddr);
    l2 += lane_xor(l2, xaddr);
    float lam;
    if (V2) {
        lam = (qrow < a.seq_q) ? a.lam[b * a.lams[0] + (int64_t)qrow * a.lams[1] + (int64_t)hout * a.lams[2]] : 0.f;
    } else {
        lam = a.lam[hout];
    }
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
        ss += lane_xor(ss, xaddr);
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

template <int D, bool V2>
hipError_t launch_fwd(const MfmaFwdArgs& a, hipStream_t stream) {
    using C = Cfg<D, V2>;
    const int pairs_per_block = V2 ? a.kv_group / 2 : 1;
    const int BM = 32 * (C::NW / pairs_per_block);
    const int n_units = V2 ? a.batch * (a.heads * 2 / a.kv_group) : a.batch * a.heads;
    const int nqt = (a.seq_q + BM - 1) / BM;
    const dim3 grid((unsigned)(nqt * n_units));
    const size_t smem = 2 * C::STAGE * sizeof(bf16);
    if (a.causal) {
        if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, true>), grid, dim3(C::NT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, true, false>), grid, dim3(C::NT), smem, stream, a);
    } else {
        if (a.epi) hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, true>), grid, dim3(C::NT), smem, stream, a);
        else hipLaunchKernelGGL((fwd_mfma_kernel<D, V2, false, false>), grid, dim3(C::NT), smem, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_v1_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream) { return launch_fwd<64, false>(a, stream); }
hipError_t launch_v2_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream) { return launch_fwd<128, true>(a, stream); }

}  // namespace diffattn
