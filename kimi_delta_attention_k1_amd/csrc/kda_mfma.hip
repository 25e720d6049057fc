// kda_mfma.hip -- bf16 matrix-core path of the KDA forward for gfx950 (CDNA4).
//
// Method: the chunkwise form of the KDA recurrence on the Doubleword page "You
// Could Have Come Up with Kimi Delta Attention", section 6, with 16-token
// chunks (FlashKDA v1 deep-dive, section 1) and the two-kernel split of the
// FlashKDA pages (deep-dive section 2): a chunk-parallel kernel (K1) and a
// per-(sequence, head) recurrence (K2).
//
// Per chunk c of one (sequence, head), with G the in-chunk prefix sum of the
// log-decay (section 6.6), K_b rows khat_i exp(G_i), Q_b rows s qhat_i exp(G_i),
// K_end rows khat_j exp(G_last - G_j) (section 6.4), R and A^qk the causal
// coefficient matrices rho, chi (sections 6.3, 6.5) and A^kk = (I+R)^-1:
//   K1:  G, R, A^kk Diag(beta), A^qk, K_b, Q_b, K_end, gamma = exp(G_last)
//   K2:  Ebar = V - K_b S_c^T               (rows v_i - S_c D_{0:i} k_i)
//        E    = A^kk Diag(beta) Ebar        (section 6.3, E = Ebar A^kk^T in columns)
//        O    = Q_b S_c^T + A^qk E          (section 6.5)
//        S_{c+1}^T = Diag(gamma) S_c^T + K_end^T E   (section 6.4)
//
// Matrix-core instruction layouts relied on (64 lanes, lane l, g = l/16):
//   16x16x32 bf16: A lane l = row l%16, 8 k values; B lane l = column l%16,
//                  the same 8 k labels; D lane l = rows 4g..4g+3, column l%16.
//   16x16x16 bf16: as above with 4 k values (k = 4g..4g+3 matches D's rows).
//   16x16x4  f32 : A lane l = row l%16, k = g; B lane l = column l%16, k = g.
// Because a D fragment has the B-operand layout of a 16x16x16 product, the
// fp32 state and the error tiles feed the next product from registers. The
// contraction order inside a 32-wide k step is a free permutation, which K1
// uses to write K_b and Q_b so that the state accumulators of two 16-row tiles
// form one 16x16x32 B operand without data movement.
#include "kda_mfma_common.h"

namespace kda {

// ---------------------------------------------------------------------------
// K1: one wave per (chunk, head). Lane l holds token l%16 and key channels
// [32 g, 32 g + 32), g = l/16, so each 16-lane row is one channel group across
// the 16 tokens of the chunk.
// ---------------------------------------------------------------------------
constexpr int kK1MaxWaves = 4;

// SG: scalar gate, g_raw is [T][H] and its one value per token and head applies
// to every key channel (Gated DeltaNet, Doubleword section 3)
// KET: also write K_end in K_b's 16x16x32 operand order (token-major) to `ket`, for
// the look-ahead recurrence
template <bool SG, bool KET>
__global__ __launch_bounds__(64 * kK1MaxWaves) void k1_mfma(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ graw,
    const uint16_t *__restrict__ braw, const int32_t *__restrict__ tok_off, const int32_t *__restrict__ chunk_off,
    int N, int H, int64_t n_c_max, float lb, float scale, char *__restrict__ units, char *__restrict__ ket)
{
    __shared__ __attribute__((aligned(16))) uint16_t sKE[kK1MaxWaves][2][kD][kC];  // K_end hi, lo as [channel][token]
    // each lane's own K_end values in K_b order (4 destination lanes x 8 elements)
    __shared__ __attribute__((aligned(16))) uint16_t sKT[KET ? kK1MaxWaves : 1][64][32];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = blockIdx.x;
    const int h = blockIdx.y * (blockDim.x >> 6) + wv;  // blockDim.x / 64 divides H
    if (c >= chunk_off[N]) return;                     // uniform over the block
    const int n = find_seq(chunk_off, N, c);
    const int t0 = tok_off[n] + (c - chunk_off[n]) * kC;
    const int len = min(kC, tok_off[n + 1] - t0);
    const int tok = lane & 15, g = lane >> 4;
    const bool valid = tok < len;

    // ---- load q, k, g_raw (32 channels each) and beta_raw; padded tokens are absent (all zero)
    float qf[32], kf[32], gf[32];
    if (valid) {
        const int64_t off = ((int64_t)(t0 + tok) * H + h) * kD + 32 * g;
        const u32x4 *pq = reinterpret_cast<const u32x4 *>(q + off);
        const u32x4 *pk = reinterpret_cast<const u32x4 *>(k + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 a = pq[i], b = pk[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[8 * i + 2 * e] = bf_lo(a[e]);
                qf[8 * i + 2 * e + 1] = bf_hi(a[e]);
                kf[8 * i + 2 * e] = bf_lo(b[e]);
                kf[8 * i + 2 * e + 1] = bf_hi(b[e]);
            }
        }
        if constexpr (SG) {
            const float gs = bf16_bits_to_f32(graw[(int64_t)(t0 + tok) * H + h]);
#pragma unroll
            for (int i = 0; i < 32; ++i) gf[i] = gs;
        } else {
            const u32x4 *pg = reinterpret_cast<const u32x4 *>(graw + off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 d = pg[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gf[8 * i + 2 * e] = bf_lo(d[e]);
                    gf[8 * i + 2 * e + 1] = bf_hi(d[e]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) qf[i] = kf[i] = gf[i] = 0.f;
    }
    const float beta =
        valid ? sigmoid_fast(bf16_bits_to_f32(braw[(int64_t)(t0 + tok) * H + h])) : 0.f;

    // ---- gate (log2 units) and in-chunk inclusive prefix sum over tokens
    const float lb2 = lb * kLog2e;
    if constexpr (SG) {  // one prefix sum serves every channel
        float x = valid ? lb2 * sigmoid_fast(gf[0]) : 0.f;
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
#pragma unroll
        for (int i = 0; i < 32; ++i) gf[i] = x;
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float x = valid ? lb2 * sigmoid_fast(gf[i]) : 0.f;
            x += row_shr<1>(x);
            x += row_shr<2>(x);
            x += row_shr<4>(x);
            x += row_shr<8>(x);
            gf[i] = x;  // G_tok (log2)
        }
    }

    // ---- L2 norms over 128 channels: 32 per lane, 4 lanes per token
    float nq = 0.f, nk = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        nq += qf[i] * qf[i];
        nk += kf[i] * kf[i];
    }
    nq += __shfl_xor(nq, 16);
    nq += __shfl_xor(nq, 32);
    nk += __shfl_xor(nk, 16);
    nk += __shfl_xor(nk, 32);
    const float rq = scale * __builtin_amdgcn_rsqf(nq + kL2Eps);  // s folded into qhat
    const float rk = __builtin_amdgcn_rsqf(nk + kL2Eps);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        qf[i] *= rq;
        kf[i] *= rk;
    }

    // ---- R = strict_tril(Diag(beta) K' K''^T), R^T, (A^qk)^T with K' = khat e^{G-Gref},
    //      K'' = khat e^{Gref-G}, Gref = G at token 7 (keeps both factors within e^{+-8|lb|}).
    //      A^qk adds straight into the outputs, so its products use bf16 hi/lo splits
    //      (fp32-level accuracy); R enters only through (I+R)^-1 and plain bf16 suffices.
    //      dn = e^{Gref-G} is kept for K_end below.
    f32x4 dR = {0.f, 0.f, 0.f, 0.f}, dRT = dR, dAQT = dR;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8 kr_h, ki_h, ki_l, qr_h, qr_l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * s + e;
            const float gref = row_bcast<7>(gf[i]);  // G of token 7, same channel
            const float up = __builtin_amdgcn_exp2f(gf[i] - gref);
            const float dn = __builtin_amdgcn_exp2f(gref - gf[i]);
            const float cl = row_bcast<15>(up);  // e^{G_last - Gref} for this channel
            // K_end = khat e^{G_last - G} = khat e^{Gref - G} e^{G_last - Gref}, to LDS as [channel][token]
            // as a bf16 hi/lo pair (about 16 bits): the update adds K_end^T E into the state
            // every chunk, and one bf16 K_end leaves a 2^-9 relative error per chunk in state
            // directions that later keys never overwrite when keys stay correlated and
            // gates barely decay
            const float ke = kf[i] * dn * cl;
            const __bf16 keh = (__bf16)ke;
            const uint16_t keb = __builtin_bit_cast(uint16_t, keh);
            sKE[wv][0][32 * g + i][tok] = keb;
            sKE[wv][1][32 * g + i][tok] = __builtin_bit_cast(uint16_t, (__bf16)(ke - (float)keh));
            if constexpr (KET) sKT[wv][lane][((i & 15) >> 2) * 8 + (i & 3) + 4 * (i >> 4)] = keb;
            const float kr = kf[i] * up, ki = kf[i] * dn, qr = qf[i] * up;
            kr_h[e] = (__bf16)kr;
            ki_h[e] = (__bf16)ki;
            ki_l[e] = (__bf16)(ki - (float)ki_h[e]);
            qr_h[e] = (__bf16)qr;
            qr_l[e] = (__bf16)(qr - (float)qr_h[e]);
        }
        dR = mma32(kr_h, ki_h, dR);
        dRT = mma32(ki_h, kr_h, dRT);
        dAQT = mma32(ki_h, qr_h, dAQT);
        dAQT = mma32(ki_l, qr_h, dAQT);
        dAQT = mma32(ki_h, qr_l, dAQT);
    }
    // D layout: row a = 4g + r, column b = tok.
    float beta_row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) beta_row[r] = __shfl(beta, 4 * g + r);
    f32x4 R, RT, AQT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int a = 4 * g + r;
        R[r] = (tok < a) ? beta_row[r] * dR[r] : 0.f;  // R[a][tok] = beta_a <k_tok|D|k_a>
        RT[r] = (a < tok) ? beta * dRT[r] : 0.f;       // R^T[a][tok] = R[tok][a]
        AQT[r] = (a <= tok) ? dAQT[r] : 0.f;           // (A^qk)^T[a][tok] = chi_{tok,a}
    }

    // ---- (A^kk)^T = (I + M)^-1 with M = R^T (strictly upper triangular), by block
    // inversion over levels of diagonal blocks of 2, 4, 8 and 16 rows: with X the inverse
    // of one level's diagonal blocks and C the part of M in the next level's off-diagonal
    // blocks, X - X C X inverts the next level's blocks. Every value formed is a block
    // of the inverse or a sum of bounded products; the doubling product
    // (I - M)(I + M^2)(I + M^4)(I + M^8) would form M^8, whose entries reach the
    // thousands for correlated keys that barely decay, and then cancel.
    auto blk = [&](int L, f32x4 x) {  // the part of x in level L's off-diagonal blocks
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int a = 4 * g + r;
            x[r] = ((a >> L) == (tok >> L) && (a >> (L - 1)) != (tok >> (L - 1))) ? x[r] : 0.f;
        }
        return x;
    };
    f32x4 Xi = eye_plus(blk(1, RT), -1.f, g, tok), XiT = eye_plus(blk(1, R), -1.f, g, tok);
#pragma unroll
    for (int L = 2; L <= 3; ++L) {  // Y = C_L Xi; Xi <- Xi - Xi Y, XiT <- XiT - Y^T XiT
        const f32x4 Y = mm16_f32(blk(L, R), Xi);
        const f32x4 Z = mm16_f32(XiT, Y), ZT = mm16_f32(Y, XiT);
        Xi -= Z;
        XiT -= ZT;
    }
    const f32x4 AT = Xi - mm16_f32(XiT, mm16_f32(blk(4, R), Xi));
    f32x4 ABT;  // (A^kk Diag(beta))^T[a][tok] = beta_a A^kk[tok][a]
#pragma unroll
    for (int r = 0; r < 4; ++r) ABT[r] = beta_row[r] * AT[r];

    char *u = units + ((int64_t)h * n_c_max + c) * kUnitBf16.bytes;
    reinterpret_cast<bf16x8 *>(u + kUnitBf16.ab)[lane] = split8(ABT);
    reinterpret_cast<bf16x8 *>(u + kUnitBf16.aq)[lane] = split8(AQT);

    // ---- K_b, Q_b (16x16x32 A-operand order); gamma = e^{G_last} from token 15's e^{G}
    float *gm = reinterpret_cast<float *>(u + kUnitBf16.gm) + 32 * g;
#pragma unroll
    for (int gp = 0; gp < 4; ++gp) {  // destination lane tok + 16 gp, k step = g
        bf16x8 kb, qb;
        float dec[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = (e < 4) ? (4 * gp + e) : (16 + 4 * gp + e - 4);
            dec[e] = __builtin_amdgcn_exp2f(gf[i]);
            kb[e] = (__bf16)(kf[i] * dec[e]);
            qb[e] = (__bf16)(qf[i] * dec[e]);
        }
        const int64_t slot = (int64_t)g * 1024 + (tok + 16 * gp) * 16;
        *reinterpret_cast<bf16x8 *>(u + kUnitBf16.kb + slot) = kb;
        *reinterpret_cast<bf16x8 *>(u + kUnitBf16.qb + slot) = qb;
        if (tok == 15) {
            *reinterpret_cast<f32x4 *>(gm + 4 * gp) = f32x4{dec[0], dec[1], dec[2], dec[3]};
            *reinterpret_cast<f32x4 *>(gm + 16 + 4 * gp) = f32x4{dec[4], dec[5], dec[6], dec[7]};
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // lane (kc = tok, g): tiles 2p and 2p+1 (channels 32p + kc and 32p + 16 + kc),
        // tokens 4g..4g+3, each tile's hi values then its lo values
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x2 h2 = *reinterpret_cast<const u32x2 *>(&sKE[wv][0][32 * p + 16 * tt + tok][4 * g]);
            const u32x2 l2 = *reinterpret_cast<const u32x2 *>(&sKE[wv][1][32 * p + 16 * tt + tok][4 * g]);
            reinterpret_cast<u32x4 *>(u + kUnitBf16.ke + p * 2048)[2 * lane + tt] = u32x4{h2[0], h2[1], l2[0], l2[1]};
        }
    }
    if constexpr (KET) {
        // lane (tok, g) owns k step g; its element group gp goes to destination lane tok + 16 gp
        char *kt = ket + ((int64_t)h * n_c_max + c) * kKetBytes + g * 1024;
#pragma unroll
        for (int gp = 0; gp < 4; ++gp)
            *reinterpret_cast<u32x4 *>(kt + (tok + 16 * gp) * 16) = *reinterpret_cast<const u32x4 *>(&sKT[wv][lane][8 * gp]);
    }
}

// ---------------------------------------------------------------------------
// K2: one workgroup per (sequence, head): 8 consumer waves, wave w owning value
// channels [16w, 16w+16), and 2 producer waves; with fewer pairs, 8 / CONS
// workgroups of CONS consumer waves per pair (K2Shape). Lane l of a consumer holds
// S^T[16t + 4g + r][16w + l%16] in accumulator tile t (t = 0..7, r = 0..3). The
// value channels evolve independently, so consumers never exchange state; they
// share each chunk's operands through LDS.
//
// The producers copy every chunk's 18944-byte workspace unit and the v rows of the
// workgroup's value columns straight from global memory into a ring of LDS slots
// with 16-byte-per-lane global-to-LDS loads, several chunks ahead, and wait with
// explicit counts of their own loads. One workgroup barrier per chunk publishes a
// slot and recycles the previous one. The barrier is a bare s_barrier: a fenced
// barrier would drain the prefetch queue every chunk.
// ---------------------------------------------------------------------------
constexpr int kVOff = 19 * 1024;  // v rows offset inside a slot
static_assert(kUnitBf16.bytes <= (size_t)kVOff, "unit must fit below the v rows");

// Workgroup shape for CONS consumer waves (8 / CONS workgroups per (sequence, head)).
// A slot holds the unit and the v rows of the workgroup's 16 CONS value columns
// (32 CONS bytes per token row, at least 1 KB). Small workgroups, which run when few
// (sequence, head) pairs share the chip, get four producer waves: the global-to-LDS
// copy rate of one wave, not memory latency, bounds their chunk rate.
template <int CONS> struct K2Shape {
    // Up to four recurrence waves get an output wave each, which forms the outputs one
    // chunk behind on its own copy of the state, off the recurrence's critical path.
    static constexpr bool split_out = CONS <= 4;
    static constexpr int consumers = split_out ? 2 * CONS : CONS;
    static constexpr int producers = CONS >= 4 ? 2 : 4;
    static constexpr int v_kb = CONS >= 2 ? CONS / 2 : 1;
    static constexpr int slot_kb = (kVOff / 1024 + v_kb + producers - 1) / producers * producers;
    static constexpr int slot_bytes = slot_kb * 1024;
    static constexpr int slots = producers == 2 ? 6 : 7;
    static constexpr int threads = 64 * (consumers + producers);
    static constexpr int kb_per_producer = slot_kb / producers;
    // chunks copied ahead of the recurrence: an output wave still reads the slot
    // of the previous chunk
    static constexpr int ahead = split_out ? slots - 2 : slots - 1;
    static constexpr int pending = (ahead - 1) * kb_per_producer;  // loads allowed in flight
    static_assert(pending <= 63, "vmcnt holds at most 63 outstanding loads");
    static constexpr int ebuf_bytes = split_out ? 2 * CONS * 1024 : 0;
    static_assert(slots * slot_bytes + ebuf_bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// RS: bf16-resident state -- the state is rounded to bf16 when it is loaded and
// after every chunk's fp32 update, as a design that keeps the on-chip state in bf16
// between updates would (FlashKDA deep-dive, section 3); it exists to measure that
// choice against the fp32 state.
template <typename TSt, int CONS, bool RS>
__global__ __launch_bounds__(K2Shape<CONS>::threads) void k2_mfma(
    const uint16_t *__restrict__ v, const TSt *s0, TSt *s1, uint16_t *__restrict__ out,
    const int32_t *__restrict__ tok_off, const int32_t *__restrict__ chunk_off, int H, int pairs, int64_t n_c_max,
    const char *__restrict__ units)
{
    using Sh = K2Shape<CONS>;
    constexpr int kGroups = 8 / CONS;  // workgroups per (sequence, head)
    __shared__ __attribute__((aligned(1024))) char lds[Sh::slots][Sh::slot_bytes];
    // E of each recurrence wave's chunk for its output wave (fp32, D layout; the output
    // wave splits it the same way), alternating by chunk parity
    __shared__ f32x4 ebuf[Sh::split_out ? 2 : 1][CONS][64];
    // the wave index is uniform over the wave: keep it scalar so role branches and
    // the address arithmetic built on it stay in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup b runs on XCD b % 8; the kGroups workgroups of one pair share an
    // XCD (and its L2), which serves the repeated unit reads.
    int pair = blockIdx.x, wbase = 0;
    if (kGroups > 1) {
        const int b = blockIdx.x;
        pair = (b & 7) + 8 * (b / (8 * kGroups));
        wbase = ((b >> 3) % kGroups) * CONS;
        if (pair >= pairs) return;  // whole workgroup: no barrier is entered
    }
    const int n = pair / H, h = pair % H;
    const int c0 = chunk_off[n], nch = chunk_off[n + 1] - c0;
    const int tb = tok_off[n], te = tok_off[n + 1];

    if (w >= Sh::consumers) {
        // ------------------------------------------------------------ producers
        if (nch == 0) return;  // uniform over the workgroup: nobody enters the barriers
        const int pw = w - Sh::consumers;
        constexpr int kKBPerProducer = Sh::kb_per_producer;
        constexpr int kProdPending = Sh::pending;
        const char *ubase = units + ((int64_t)h * n_c_max + c0) * kUnitBf16.bytes;
        const char *vb = reinterpret_cast<const char *>(v);
        auto copy_chunk = [&](int j, int slot) {
            j = min(j, nch - 1);  // past the end: re-read the last chunk into a free slot
            const char *u = ubase + (int64_t)j * kUnitBf16.bytes;
#pragma unroll
            for (int i = 0; i < kKBPerProducer; ++i) {
                const int b = pw * kKBPerProducer + i;  // which KB of the slot
                const char *src;
                if (b < kVOff / 1024) {
                    const int off = b * 1024 + lane * 16;
                    src = u + (off < (int)kUnitBf16.bytes ? off : 0);
                } else if (b < kVOff / 1024 + Sh::v_kb) {
                    // 16-byte piece `seg` of the v rows: token row seg / (2 CONS), columns
                    // 16 wbase + 8 (seg % (2 CONS)) ..; a 1 KB region wider than the rows
                    // (CONS = 1) repeats them
                    const int seg = (b - kVOff / 1024) * 64 + lane;
                    const int r = (seg / (2 * CONS)) & 15;
                    const int row = min(tb + j * kC + r, te - 1);
                    src = vb + (((int64_t)row * H + h) * kD + 16 * wbase + 8 * (seg % (2 * CONS))) * 2;
                } else {
                    src = u;  // filler: keeps every producer at the same load count
                }
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(&lds[slot][b * 1024]), 16, 0, 0);
            }
        };
#pragma unroll
        for (int s = 0; s < Sh::ahead; ++s) copy_chunk(s, s);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kProdPending) : "memory");  // chunk 0 landed
        bar_sync();
#pragma unroll 1
        for (int j = 0; j < nch; ++j) {
            copy_chunk(j + Sh::ahead, (j + Sh::ahead) % Sh::slots);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kProdPending) : "memory");  // chunk j+1 landed
            bar_sync();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // nothing in flight into LDS at exit
        return;
    }

    // ---------------------------------------------------------------- consumers
    const bool out_wave = Sh::split_out && w >= CONS;
    const int wc = out_wave ? w - CONS : w;  // value-column tile within the workgroup
    const int g = lane >> 4, vcol = 16 * (wbase + wc) + (lane & 15);
    const int64_t sbase = (((int64_t)n * H + h) * kD + vcol) * kD + 4 * g;
    f32x4 st[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s0 != nullptr) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st[t] = ld_state4(s0 + sbase + 16 * t);
    }
    if constexpr (RS) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st[t] = round_bf16x4(st[t]);
    }
    if (nch > 0) bar_sync();
    if constexpr (Sh::split_out) {
        // state -> bf16 B operands (tiles 2p, 2p+1 form k step p)
        auto cast_state = [&](bf16x8(&sb)[4]) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sb[p][r] = (__bf16)st[2 * p][r];
                    sb[p][4 + r] = (__bf16)st[2 * p + 1][r];
                }
            }
        };
        // S^T <- Diag(gamma) S^T + K_end^T E, K_end = hi + lo and E = E_hi + E_lo:
        // [hi | lo] x [E_hi ; E_hi] + [hi | lo] x [E_lo ; E_lo], two 16x16x32 products
        auto update = [&](const char *L, bf16x4 e_h, bf16x4 e_l) {
            const bf16x8 ehh = cat8(e_h, e_h), ell = cat8(e_l, e_l);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.ke + (t >> 1) * 2048 + lane * 32 + (t & 1) * 16);
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(L + kUnitBf16.gm + (16 * t + 4 * g) * 4);
                st[t] = mma32(k8, ell, mma32(k8, ehh, st[t] * gm));
                if constexpr (RS) st[t] = round_bf16x4(st[t]);
            }
        };
        if (!out_wave) {
            // ------------------------------------------------ recurrence wave
#pragma unroll 1
            for (int j = 0; j < nch; ++j) {
                const char *L = lds[j % Sh::slots];
                const int t0 = tb + j * kC;
                const int len = min(kC, te - t0);
                bf16x8 sb[4];
                cast_state(sb);
                f32x4 xk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.kb + p * 1024 + lane * 16);
                    xk = mma32(kb, sb[p], xk);
                }
                // Ebar = V - K_b S^T ; E = (A^kk Diag(beta)) Ebar with split operands
                f32x4 eb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 4 * g + r;
                    const uint16_t vr =
                        *reinterpret_cast<const uint16_t *>(L + kVOff + tr * (32 * CONS) + (vcol - 16 * wbase) * 2);
                    eb[r] = (tr < len ? bf16_bits_to_f32(vr) : 0.f) - xk[r];
                }
                bf16x4 eb_h, eb_l, e_h, e_l;
                split4(eb, eb_h, eb_l);
                const bf16x8 ab = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.ab + lane * 16);
                f32x4 E = {0.f, 0.f, 0.f, 0.f};
                E = mma32(ab, cat8(eb_h, eb_h), E);
                E = mma32(ab, cat8(eb_l, eb_l), E);
                split4(E, e_h, e_l);
                // the output wave gets E in fp32 and splits it itself (a variant that handed
                // over the bf16 hi/lo registers gave wrong outputs; it chained products of
                // two shapes, which the note at mma16 explains)
                ebuf[j & 1][wc][lane] = E;
                update(L, e_h, e_l);
                // the E tile is in LDS before the barrier publishes it
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                bar_sync();
            }
            if (s1) {
#pragma unroll
                for (int t = 0; t < 8; ++t) st_state4(s1 + sbase + 16 * t, st[t]);
            }
        } else {
            // ---------------------------------------------------- output wave
            // chunk c's outputs from the state before chunk c and the E tile its
            // recurrence wave published; then the same state update, so this copy of
            // the state stays bitwise equal to the recurrence wave's
            auto out_step = [&](int c, bool upd) {
                const char *L = lds[c % Sh::slots];
                const int t0 = tb + c * kC;
                const int len = min(kC, te - t0);
                bf16x8 sb[4];
                cast_state(sb);
                f32x4 xq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.qb + p * 1024 + lane * 16);
                    xq = mma32(qb, sb[p], xq);
                }
                bf16x4 e_h, e_l;
                split4(ebuf[c & 1][wc][lane], e_h, e_l);
                // O = Q_b S^T + A^qk E
                const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.aq + lane * 16);
                f32x4 O = mma32(aq, cat8(e_h, e_h), xq);
                O = mma32(aq, cat8(e_l, e_l), O);
                uint16_t *orow = out + ((int64_t)(t0 + 4 * g) * H + h) * kD + vcol;
                const int64_t rstride = (int64_t)H * kD;
                if (len == kC) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) orow[r * rstride] = __builtin_bit_cast(uint16_t, (__bf16)O[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r < len) orow[r * rstride] = __builtin_bit_cast(uint16_t, (__bf16)O[r]);
                }
                if (upd) update(L, e_h, e_l);
            };
#pragma unroll 1
            for (int j = 0; j < nch; ++j) {
                if (j > 0) out_step(j - 1, true);
                // this wave's LDS reads (the E tile the recurrence wave rewrites two
                // barriers on, the unit's slot) are complete before the barrier
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                bar_sync();
            }
            if (nch > 0) out_step(nch - 1, false);
        }
        return;
    }
#pragma unroll 1
    for (int j = 0; j < nch; ++j) {
        const char *L = lds[j % Sh::slots];
        const int t0 = tb + j * kC;
        const int len = min(kC, te - t0);

        // state -> bf16 B operands (tiles 2p, 2p+1 form k step p)
        bf16x8 sb[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sb[p][r] = (__bf16)st[2 * p][r];
                sb[p][4 + r] = (__bf16)st[2 * p + 1][r];
            }
        }
        f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = xk;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.kb + p * 1024 + lane * 16);
            const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.qb + p * 1024 + lane * 16);
            xk = mma32(kb, sb[p], xk);
            xq = mma32(qb, sb[p], xq);
        }
        // Ebar = V - K_b S^T ; E = (A^kk Diag(beta)) Ebar with split operands
        f32x4 eb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tr = 4 * g + r;
            const uint16_t vr =
                *reinterpret_cast<const uint16_t *>(L + kVOff + tr * (32 * CONS) + (vcol - 16 * wbase) * 2);
            eb[r] = (tr < len ? bf16_bits_to_f32(vr) : 0.f) - xk[r];
        }
        // A operands arrive as {hi, lo}: [hi | lo] x [x_hi ; x_hi] + [hi | lo] x [x_lo ; x_lo]
        // is the split product (hi + lo)(x_hi + x_lo) in two 16x16x32 instructions.
        bf16x4 eb_h, eb_l, e_h, e_l;
        split4(eb, eb_h, eb_l);
        const bf16x8 ab = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.ab + lane * 16);
        f32x4 E = {0.f, 0.f, 0.f, 0.f};
        E = mma32(ab, cat8(eb_h, eb_h), E);
        E = mma32(ab, cat8(eb_l, eb_l), E);
        split4(E, e_h, e_l);
        // O = Q_b S^T + A^qk E
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.aq + lane * 16);
        f32x4 O = mma32(aq, cat8(e_h, e_h), xq);
        O = mma32(aq, cat8(e_l, e_l), O);
        uint16_t *orow = out + ((int64_t)(t0 + 4 * g) * H + h) * kD + vcol;
        const int64_t rstride = (int64_t)H * kD;
        if (len == kC) {
#pragma unroll
            for (int r = 0; r < 4; ++r) orow[r * rstride] = __builtin_bit_cast(uint16_t, (__bf16)O[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r < len) orow[r * rstride] = __builtin_bit_cast(uint16_t, (__bf16)O[r]);
        }
        // S^T <- Diag(gamma) S^T + K_end^T E, K_end = hi + lo and E = E_hi + E_lo:
        // [hi | lo] x [E_hi ; E_hi] + [hi | lo] x [E_lo ; E_lo]
        const bf16x8 ehh = cat8(e_h, e_h), ell = cat8(e_l, e_l);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.ke + (t >> 1) * 2048 + lane * 32 + (t & 1) * 16);
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(L + kUnitBf16.gm + (16 * t + 4 * g) * 4);
            st[t] = mma32(k8, ell, mma32(k8, ehh, st[t] * gm));
            if constexpr (RS) st[t] = round_bf16x4(st[t]);
        }
        // this wave's reads of the slot are complete before it may be refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bar_sync();  // this chunk's slot may be refilled; chunk j+1 is published
    }
    if (s1) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st_state4(s1 + sbase + 16 * t, st[t]);
    }
}


// ---------------------------------------------------------------------------
// Look-ahead recurrence for few (sequence, head) pairs, where the chain of one
// chunk's dependent steps, not throughput, sets the pace. With
//   S_c^T = Diag(gamma_{c-1}) S_{c-1}^T + K_end,{c-1}^T E_{c-1},
// the product the next E needs splits as
//   K_b,c S_c^T = P_c + M_c E_{c-1},  P_c = K_b,c (Diag(gamma_{c-1}) S_{c-1}^T),
//   M_c = K_b,c K_end,{c-1}^T,
// where P_c needs only the previous state. Each 16-column tile gets four waves:
//   E wave    : E_c from P_c + M_c E_{c-1} (the only chain from one E to the next)
//   state waves (2): keys 0-63 and 64-127 of the state; each applies the update
//               with E_{c-1}, then forms its halves of Q_b,c S_c^T and P_{c+1}
//   output wave: M_{c+1} from K_end in K_b order (written by K1), and the outputs
//               of chunk c-1 from Q_b S^T and E
// Everything passes through LDS between barriers; each value is produced in one
// iteration and used in the next. The state waves run one iteration ahead (an
// extra first iteration forms P_0).
// ---------------------------------------------------------------------------
template <int CONS> struct KLShape {
    static constexpr int producers = 4;
    static constexpr int unit_kb = kVOff / 1024;                  // unit, then K_end in K_b order
    static constexpr int v_kb = 1;                                // v rows of 16 CONS columns
    static constexpr int slot_kb = unit_kb + 4 + v_kb;            // 24
    static constexpr int slot_bytes = slot_kb * 1024;
    static constexpr int slots = CONS == 1 ? 6 : 5;
    static constexpr int consumers = 4 * CONS;
    static constexpr int threads = 64 * (consumers + producers);
    static constexpr int kb_per_producer = slot_kb / producers;
    // chunk c + ahead is copied while chunks c - 1 .. c + 1 are read
    static constexpr int ahead = slots - 2;
    static constexpr int pending = (ahead - 2) * kb_per_producer;  // chunk c + 2 landed at barrier c + 1
    static constexpr int xbuf_bytes = 2 * CONS * 6 * 1024;        // E, M, 2 x P, 2 x Q_b S^T, by parity
    static_assert(slot_kb % producers == 0, "producers split a slot evenly");
    static_assert(v_kb * 1024 >= 32 * CONS * kC, "v rows fit");
    static_assert(pending <= 63 && ahead >= 3, "copy pipeline");
    static_assert(slots * slot_bytes + xbuf_bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

template <typename TSt, int CONS>
__global__ __launch_bounds__(KLShape<CONS>::threads) void k2_look(
    const uint16_t *__restrict__ v, const TSt *s0, TSt *s1, uint16_t *__restrict__ out,
    const int32_t *__restrict__ tok_off, const int32_t *__restrict__ chunk_off, int H, int pairs, int64_t n_c_max,
    const char *__restrict__ units, const char *__restrict__ kets)
{
    using Sh = KLShape<CONS>;
    constexpr int kGroups = 8 / CONS;
    __shared__ __attribute__((aligned(1024))) char lds[Sh::slots][Sh::slot_bytes];
    __shared__ f32x4 ebuf[2][CONS][64], mbuf[2][CONS][64], pbuf[2][2][CONS][64], xqbuf[2][2][CONS][64];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int pair = (b & 7) + 8 * (b / (8 * kGroups));
    const int wbase = ((b >> 3) % kGroups) * CONS;
    if (pair >= pairs) return;  // whole workgroup: no barrier is entered
    const int n = pair / H, h = pair % H;
    const int c0 = chunk_off[n], nch = chunk_off[n + 1] - c0;
    const int tb = tok_off[n], te = tok_off[n + 1];
    constexpr int kKet = Sh::unit_kb * 1024;  // K_end in K_b order, inside a slot
    constexpr int kV = kKet + 4096;           // v rows
    const int role = w / CONS, wc = w % CONS;  // 0: E wave, 1-2: state waves, 3: output wave, 4+: producers
    const int g = lane >> 4, vcol = 16 * (wbase + wc) + (lane & 15);
    if (nch == 0) {  // uniform over the workgroup: no barrier is entered
        if ((role == 1 || role == 2) && s1) {
            const int64_t sb0 = (((int64_t)n * H + h) * kD + vcol) * kD + 64 * (role - 1) + 4 * g;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                st_state4(s1 + sb0 + 16 * t, s0 ? ld_state4(s0 + sb0 + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f});
        }
        return;
    }

    if (w >= Sh::consumers) {
        // ------------------------------------------------------------ producers
        const int pw = w - Sh::consumers;
        constexpr int kKB = Sh::kb_per_producer;
        const char *ubase = units + ((int64_t)h * n_c_max + c0) * kUnitBf16.bytes;
        const char *kbase = kets + ((int64_t)h * n_c_max + c0) * kKetBytes;
        const char *vb = reinterpret_cast<const char *>(v);
        auto copy_chunk = [&](int j, int slot) {
            j = min(j, nch - 1);  // past the end: re-read the last chunk into a free slot
            const char *u = ubase + (int64_t)j * kUnitBf16.bytes;
#pragma unroll
            for (int i = 0; i < kKB; ++i) {
                const int kb = pw * kKB + i;  // which KB of the slot
                const char *src;
                if (kb < Sh::unit_kb) {
                    const int off = kb * 1024 + lane * 16;
                    src = u + (off < (int)kUnitBf16.bytes ? off : 0);
                } else if (kb < Sh::unit_kb + 4) {
                    src = kbase + (int64_t)j * kKetBytes + (kb - Sh::unit_kb) * 1024 + lane * 16;
                } else {
                    // 16-byte piece `lane` of the v rows: token row lane / (2 CONS), columns
                    // 16 wbase + 8 (lane % (2 CONS)) ..; lanes past the rows repeat them
                    const int r = (lane / (2 * CONS)) & 15;
                    const int row = min(tb + j * kC + r, te - 1);
                    src = vb + (((int64_t)row * H + h) * kD + 16 * wbase + 8 * (lane % (2 * CONS))) * 2;
                }
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(&lds[slot][kb * 1024]), 16, 0, 0);
            }
        };
#pragma unroll
        for (int sl = 0; sl < Sh::ahead; ++sl) copy_chunk(sl, sl);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Sh::pending) : "memory");  // chunks 0 and 1 landed
        bar_sync();
        bar_sync();  // the state waves' first iteration
#pragma unroll 1
        for (int j = 0; j < nch; ++j) {
            copy_chunk(j + Sh::ahead, (j + Sh::ahead) % Sh::slots);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Sh::pending) : "memory");  // chunk j+2 landed
            bar_sync();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // nothing in flight into LDS at exit
        return;
    }

    bar_sync();

    if (role == 0) {
        // ---------------------------------------------------------------- E wave
        bar_sync();  // the state waves form P_0
        bf16x4 ep_h = {}, ep_l = {};  // previous chunk's E, split
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            const char *L = lds[c % Sh::slots];
            const int t0 = tb + c * kC, len = min(kC, te - t0);
            f32x4 xk = pbuf[c & 1][0][wc][lane] + pbuf[c & 1][1][wc][lane];
            if (c > 0) {  // + M E_prev in split operands
                bf16x4 m_h, m_l;
                split4(mbuf[c & 1][wc][lane], m_h, m_l);
                const bf16x8 m_hl = cat8(m_h, m_l);
                xk = mma32(m_hl, cat8(ep_h, ep_h), xk);
                xk = mma32(m_hl, cat8(ep_l, ep_l), xk);
            }
            f32x4 eb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 4 * g + r;
                const uint16_t vr =
                    *reinterpret_cast<const uint16_t *>(L + kV + tr * (32 * CONS) + 32 * wc + 2 * (lane & 15));
                eb[r] = (tr < len ? bf16_bits_to_f32(vr) : 0.f) - xk[r];
            }
            bf16x4 eb_h, eb_l;
            split4(eb, eb_h, eb_l);
            const bf16x8 ab = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.ab + lane * 16);
            f32x4 E = {0.f, 0.f, 0.f, 0.f};
            E = mma32(ab, cat8(eb_h, eb_h), E);
            E = mma32(ab, cat8(eb_l, eb_l), E);
            ebuf[c & 1][wc][lane] = E;
            split4(E, ep_h, ep_l);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            bar_sync();
        }
        return;
    }

    if (role <= 2) {
        // ------------------------------------------------------------ state waves
        // tiles 4 i .. 4 i + 3 of the state (keys 64 i .. 64 i + 63), k steps 2 i, 2 i + 1
        const int i = role - 1;
        const int64_t sbase = (((int64_t)n * H + h) * kD + vcol) * kD + 64 * i + 4 * g;
        f32x4 st[4], dec[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) st[t] = s0 ? ld_state4(s0 + sbase + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        // half of Y X^T over this wave's 64 keys, X in fp32 tiles
        auto half_prod = [&](const char *L, int off, const f32x4 (&x)[4]) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                bf16x8 sb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sb[r] = (__bf16)x[2 * pp][r];
                    sb[4 + r] = (__bf16)x[2 * pp + 1][r];
                }
                a = mma32(*reinterpret_cast<const bf16x8 *>(L + off + (2 * i + pp) * 1024 + lane * 16), sb, a);
            }
            return a;
        };
        // P_0 = K_b,0 S_0^T
        pbuf[0][i][wc][lane] = half_prod(lds[0], kUnitBf16.kb, st);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bar_sync();
        // S^T <- Diag(gamma) S^T + K_end^T E for chunk cp, from the decayed state
        auto update = [&](int cp) {
            const char *Lp = lds[cp % Sh::slots];
            bf16x4 e_h, e_l;
            split4(ebuf[cp & 1][wc][lane], e_h, e_l);
            const bf16x8 ehh = cat8(e_h, e_h), ell = cat8(e_l, e_l);
            // K_end = hi + lo: [hi | lo] x [E_hi ; E_hi] + [hi | lo] x [E_lo ; E_lo]
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int tg = 4 * i + t;  // the state tile of this wave's keys
                const bf16x8 k8 =
                    *reinterpret_cast<const bf16x8 *>(Lp + kUnitBf16.ke + (tg >> 1) * 2048 + lane * 32 + (tg & 1) * 16);
                st[t] = mma32(k8, ell, mma32(k8, ehh, dec[t]));
            }
        };
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            const char *L = lds[c % Sh::slots];
            if (c > 0) update(c - 1);
            xqbuf[c & 1][i][wc][lane] = half_prod(L, kUnitBf16.qb, st);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dec[t] = st[t] * *reinterpret_cast<const f32x4 *>(L + kUnitBf16.gm + (64 * i + 16 * t + 4 * g) * 4);
            if (c + 1 < nch) pbuf[(c + 1) & 1][i][wc][lane] = half_prod(lds[(c + 1) % Sh::slots], kUnitBf16.kb, dec);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            bar_sync();
        }
        update(nch - 1);
        if (s1) {
#pragma unroll
            for (int t = 0; t < 4; ++t) st_state4(s1 + sbase + 16 * t, st[t]);
        }
        return;
    }

    // ---------------------------------------------------------------- output wave
    bar_sync();  // the state waves form P_0
    auto out_step = [&](int c) {
        const char *L = lds[c % Sh::slots];
        const int t0 = tb + c * kC, len = min(kC, te - t0);
        bf16x4 e_h, e_l;
        split4(ebuf[c & 1][wc][lane], e_h, e_l);
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(L + kUnitBf16.aq + lane * 16);
        f32x4 O = mma32(aq, cat8(e_h, e_h), xqbuf[c & 1][0][wc][lane] + xqbuf[c & 1][1][wc][lane]);
        O = mma32(aq, cat8(e_l, e_l), O);
        uint16_t *orow = out + ((int64_t)(t0 + 4 * g) * H + h) * kD + vcol;
        const int64_t rstride = (int64_t)H * kD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r < len) orow[r * rstride] = __builtin_bit_cast(uint16_t, (__bf16)O[r]);
    };
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) {
            // M_{c+1}^T = K_end,c K_b,{c+1}^T, whose D layout is M_{c+1} in A-operand order
            const char *L = lds[c % Sh::slots];
            const char *Ln = lds[(c + 1) % Sh::slots];
            f32x4 mt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p)
                mt = mma32(*reinterpret_cast<const bf16x8 *>(L + kKet + p * 1024 + lane * 16),
                           *reinterpret_cast<const bf16x8 *>(Ln + kUnitBf16.kb + p * 1024 + lane * 16), mt);
            mbuf[(c + 1) & 1][wc][lane] = mt;
        }
        if (c > 0) out_step(c - 1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bar_sync();
    }
    out_step(nch - 1);
}

// chunk kernel: waves (one per (chunk, head) unit) per workgroup, a divisor of H
static int k1_waves(int H) { return (H % 4 == 0) ? 4 : (H % 2 == 0 ? 2 : 1); }

// recurrence workgroups: 8 / CONS per (sequence, head) pair, the pair count padded
// to a multiple of 8 when a pair takes several
template <int CONS> static int64_t k2_grid(int64_t pairs)
{
    constexpr int groups = 8 / CONS;
    return groups == 1 ? pairs : (pairs + 7) / 8 * 8 * groups;
}

hipError_t launch_prep_mfma(const Problem &p, hipStream_t s)
{
    if (p.n_c_max == 0) return hipSuccess;
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    const int wpb = k1_waves(p.H);
    const bool look = use_lookahead(p.N, p.H, false, p.bf16_resident);
    auto kern = p.scalar_gate ? (look ? k1_mfma<true, true> : k1_mfma<true, false>)
                              : (look ? k1_mfma<false, true> : k1_mfma<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)p.n_c_max, p.H / wpb), dim3(64 * wpb), 0, s, (const uint16_t *)p.q,
                       (const uint16_t *)p.k, (const uint16_t *)p.g, (const uint16_t *)p.beta, tok, chk, (int)p.N,
                       p.H, p.n_c_max, p.lb, p.scale, p.ws + p.lay.units, look ? p.ws + p.lay.ket : nullptr);
    return hipGetLastError();
}

template <typename TSt, int CONS, bool RS>
static hipError_t launch_k2(const Problem &p, hipStream_t s)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    const int pairs = (int)(p.N * p.H);
    const unsigned grid = (unsigned)k2_grid<CONS>(pairs);
    hipLaunchKernelGGL((k2_mfma<TSt, CONS, RS>), dim3(grid), dim3(K2Shape<CONS>::threads), 0, s, (const uint16_t *)p.v,
                       (const TSt *)p.s0, (TSt *)p.s1, (uint16_t *)p.out, tok, chk, p.H, pairs, p.n_c_max,
                       (const char *)(p.ws + p.lay.units));
    return hipGetLastError();
}

// Consumer waves per workgroup: the largest that still puts about one
// workgroup on every one of the 256 compute units.
template <typename TSt, int CONS>
static hipError_t launch_look(const Problem &p, hipStream_t s)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    const int pairs = (int)(p.N * p.H);
    const unsigned grid = (unsigned)((pairs + 7) / 8 * 8 * (8 / CONS));
    hipLaunchKernelGGL((k2_look<TSt, CONS>), dim3(grid), dim3(KLShape<CONS>::threads), 0, s, (const uint16_t *)p.v,
                       (const TSt *)p.s0, (TSt *)p.s1, (uint16_t *)p.out, tok, chk, p.H, pairs, p.n_c_max,
                       (const char *)(p.ws + p.lay.units), (const char *)(p.ws + p.lay.ket));
    return hipGetLastError();
}

template <typename TSt, bool RS>
static hipError_t launch_recur_mfma_t(const Problem &p, hipStream_t s)
{
    const int64_t pairs = p.N * p.H;
    if (!RS && use_lookahead(p.N, p.H, false, false)) {
        return pairs >= 48 ? launch_look<TSt, 2>(p, s) : launch_look<TSt, 1>(p, s);
    }
    if (pairs >= 192) return launch_k2<TSt, 8, RS>(p, s);
    if (pairs >= 96) return launch_k2<TSt, 4, RS>(p, s);
    if (pairs >= 48) return launch_k2<TSt, 2, RS>(p, s);
    return launch_k2<TSt, 1, RS>(p, s);
}

bool fits_split(const Problem &p)
{
    const int wpb = k1_waves(p.H);
    if (!grid_fits(p.n_c_max, p.H / wpb, 64 * wpb)) return false;
    const int64_t pairs = p.N * p.H, padded = (pairs + 7) / 8 * 8;
    if (!p.bf16_resident && use_lookahead(p.N, p.H, false, false))
        return pairs >= 48 ? grid_fits(padded * 4, 1, KLShape<2>::threads) : grid_fits(padded * 8, 1, KLShape<1>::threads);
    if (pairs >= 192) return grid_fits(k2_grid<8>(pairs), 1, K2Shape<8>::threads);
    if (pairs >= 96) return grid_fits(k2_grid<4>(pairs), 1, K2Shape<4>::threads);
    if (pairs >= 48) return grid_fits(k2_grid<2>(pairs), 1, K2Shape<2>::threads);
    return grid_fits(k2_grid<1>(pairs), 1, K2Shape<1>::threads);
}

hipError_t launch_recur_mfma(const Problem &p, hipStream_t s)
{
    if (p.bf16_resident)
        return p.st_bf16 ? launch_recur_mfma_t<uint16_t, true>(p, s) : launch_recur_mfma_t<float, true>(p, s);
    return p.st_bf16 ? launch_recur_mfma_t<uint16_t, false>(p, s) : launch_recur_mfma_t<float, false>(p, s);
}

}  // namespace kda
