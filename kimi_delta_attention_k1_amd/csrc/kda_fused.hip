// kda_fused.hip -- single-pass bf16 KDA forward for gfx950: one workgroup per
// (sequence, head) builds each chunk's operands in LDS and runs the recurrence
// on them, so the only HBM traffic is the inputs, the outputs and the states.
//
// Same mathematics as the two-kernel path (Doubleword page "You Could Have
// Come Up with Kimi Delta Attention", section 6; see kda_mfma.hip): per chunk
// G (in-chunk prefix sums of the log-decay, 6.6), rho and chi (6.3, 6.5),
// A^kk = (I + R)^-1, then E = A^kk Diag(beta)(V - K_b S^T), O = Q_b S^T + A^qk E
// and S^T <- Diag(gamma) S^T + K_end^T E (6.4).
//
// Workgroup: 4 consumer waves (the recurrence; wave w owns value channels [32w,
// 32w+32) as two 16-wide column tiles, so every operand read from LDS serves two
// tiles), 4 stage-A waves (wave m owns key channels [32m, 32m+32)) and 3 stage-B waves:
// 8 and 10 (14 in the segmented form, after its 4 transfer-run waves) invert the even
// and the odd chunks, 9 ("role 1") forms A^qk and beta. Waves w, w+4, w+8 (and w+12)
// share a SIMD, so the two inverse waves sit on different SIMDs. Time advances in ticks
// separated by one workgroup barrier; chunk c is handled at
//   tick c    : stage A -- gate, prefix sums, decays; the wave's channel slices of
//               K_b / Q_b / K_inv / K_end (hi, lo), gamma and v into prepared slot
//               c % 4; consumer waves 3 and 1 -- the per-token scales rk = 1/|k| and
//               s rq = s/|q| of chunk c from the raw inputs (the diagonals of the raw
//               rows' Gram matrices); role 1 -- its beta
//   tick c+1  : stage B -- contracts the operands over the 128 channels; role 1
//               forms (A^qk)^T; the chunk's inverse wave forms R, R^T and the
//               first levels of the block inversion of I + R
//   tick c+2  : the inverse wave completes (A^kk Diag(beta))^T into slot c % 4
//   tick c+3  : consumers run the recurrence step on slot c % 4.
// Each stage-A wave streams its channel slices of q, k, g_raw, v and beta_raw into a
// kFIn-slot ring with global-to-LDS loads and waits on exact counts of its own loads;
// a ring slot is refilled one tick after its chunk's stage-A tick, since the consumers
// and stage B read it during that tick.
//
// L2 normalisation is deferred: stage A works on raw q, k; consumer waves 3 and 1 form
// rk and s rq (the read scale s folded in) a tick ahead of stage B, which folds them into R,
// (A^kk Diag(beta))^T and (A^qk)^T; the consumers scale K_b S^T by rk and Q_b S^T by
// rq per row. The recurrence then runs on
// E' = Diag(rk) E, which is exactly what the state update needs with the raw
// K_end (K_end^T E = K_end_raw^T E'), and A^qk / Diag(rk) applied to E' gives
// the same outputs.
#include <type_traits>

#include "kda_mfma_common.h"

namespace kda {

constexpr int kFCons = 4;  // consumer waves (32 value channels each)
constexpr int kFPrep = 4;  // stage-A waves (32 key channels each)
constexpr int kAW = 32;    // key channels per stage-A wave
constexpr int kNE = 8;     // key channels per stage-A lane
// 4 consumer, 4 stage-A and 3 stage-B waves; the segmented form adds 4 transfer-run waves
template <bool SEG> constexpr int f_threads() { return 64 * (kFCons + kFPrep + 3 + (SEG ? kFCons : 0)); }
constexpr int kFIn = 3;     // input-ring slots per stage-A wave (two chunks in flight)
constexpr int kFSlots = 4;  // prepared-chunk slots (stage A steps through them unrolled)
constexpr int kFDma = 5;    // global-to-LDS loads per chunk per stage-A wave: q, k, g_raw, v, beta
// a ring slot is refilled one tick after its chunk's stage-A tick (consumer waves 1 and 3
// read the raw q and k, stage B role 1 the beta_raw, of chunk c from the rings during tick c),
// so kFIn - 1 chunks are in flight: waiting for chunk c + 1 at the end of tick c leaves
// (kFIn - 2) chunks' loads outstanding
constexpr int kFPending = (kFIn - 2) * kFDma;
static_assert(kFPending <= 63, "vmcnt holds at most 63 outstanding loads");

// prepared slot: the chunk's operands in the consumers' matrix-core lane order (1 KB
// per 16 x 32 or 32 x 16 block, swizzled), which stage B also contracts:
//   KB  K_b = k e^{G - r}   (16x16x32 A order, k step m = key channels [32m, 32m+32))
//   QB  Q_b = q e^{G - r}   (same order)
//   KE  K_end = k e^{G_last - G} as a bf16 hi/lo pair (about 16 bits), 2 KB per tile
//       pair m: lane L's 32 bytes hold, for tiles 2m and 2m+1, four tokens' hi values
//       then the same tokens' lo values (16x16x16 A order for each half, so one 16-byte
//       read is a 16x16x32 operand [hi | lo]). The update K_end^T E' adds into the
//       state every chunk, so a one-bf16 K_end would leave a 2^-9 relative error per
//       chunk in state directions that later keys never overwrite: with correlated
//       keys and gates that barely decay that grew past the bf16 bound
//   AB  (Diag(rk) A^kk Diag(beta))^T, AQ (A^qk)^T as bf16 hi/lo pairs; GM gamma = e^{G_last}
//   SC  rk[16], s*rq[16]
//   KI  K_inv = k e^{r - G}  (KB's order)
//   V   the v tile [16][128] bf16, rows kVRow bytes apart
//   ER  e^{r} per key channel (token-7 reference only; the consumers scale their bf16
//       state operand by it)
// with r = 0 (decays from the chunk start, CSR) or r = G of the chunk's token 7.
constexpr int kPKB = 0, kPQB = 4096, kPKE = 8192, kPAB = 16384, kPAQ = 17408, kPGM = 18432;
constexpr int kPSC = 18944;
constexpr int kPKI = 19072;
constexpr int kPV = kPKI + 4096;
constexpr int kVRow = 272;  // 256 + 16: row r starts 4 r banks further, so row-wise
                            // 16-byte writes and column-wise reads spread over the banks
constexpr int kPER = kPV + kC * kVRow;
template <bool CSR> constexpr int slot_bytes() { return kPER + (CSR ? 0 : 512); }
// per-stage-A-wave input slot: q, k, g_raw, v as [16 rows][32 channels] bf16, then
// beta_raw as one aligned dword per token (lanes 0-15; the token's element in its low or
// high half); a scalar g_raw takes the same dword form at the start of its block
constexpr int kIQ = 0, kIK = 1024, kIG = 2048, kIV = 3072, kIB = 4096, kIBytes = 4160;
constexpr int kXBeta = 0, kXBytes = 64;  // per-parity buffer: the chunk's beta, formed a tick ahead
template <bool CSR> constexpr int lds_bytes()
{
    return kFSlots * slot_bytes<CSR>() + kFPrep * kFIn * kIBytes + 2 * kXBytes;
}
static_assert(lds_bytes<false>() <= 160 * 1024 && lds_bytes<true>() <= 160 * 1024, "LDS budget of one workgroup");
static_assert(slot_bytes<false>() % 128 == 0 && slot_bytes<true>() % 128 == 0 && kIBytes % 64 == 0 &&
                  kPKI % 16 == 0 && kPV % 16 == 0,
              "16-byte aligned LDS blocks");

// 16-byte slot of lane L in a 1 KB operand block: L with its low three bits XORed with
// bits 3-5. The consumers' 16-byte reads still cover all banks in every group of eight
// lanes, and stage A's scattered 2- and 8-byte writes spread over the banks.
__device__ __forceinline__ int swz(int L) { return L ^ ((L >> 3) & 7); }

// barrier that first completes this wave's own LDS traffic (not its global loads)
__device__ __forceinline__ void tick_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// SG: scalar gate, g_raw is [T][H] and its one value per token and head applies to
// every key channel (Gated DeltaNet, Doubleword section 3)
//
// SEG: one workgroup per (time segment, head) instead of per (sequence, head); a
// sequence's chunks are cut into segments of seg_len chunks, the first one seg_first
// chunks long (segment g of sequence
// n is the g-th entry after seg_off[n]). The state entering a segment is not known
// yet, so the segment runs twice over the same prepared chunks, and the state
// recurrence being linear in (S, v) makes the two runs add up to the true one:
//   waves 0-3  : from S = 0 (segment 0: the initial state) with the inputs v,
//                writing the outputs o0 to `out` and the final state S0 to sfin;
//   waves 10-13: from S = I with v = 0, i.e. the key-space transfer of the
//                segment, writing y_t = Phi_t (s qhat_t) to ybuf and the segment's
//                transfer Phi to phi.
// With S_in the true incoming state, S_t = S_in Phi_t + S0_t, hence
// o_t = o0_t + S_in y_t; the scan and correction kernels (kda_seg.hip) finish it.
// Segment 0 starts from the known initial state, so its waves 10-13 only keep
// the barrier count.
//
// CSR: in-chunk decays referenced to the chunk start (lower_bound >= -5). Then
// |G| <= 16 |lb| <= 80 in natural-log units, so e^G and e^-G, and the bf16 operands
// k e^G, q e^G and k e^-G, stay inside fp32's and bf16's normal range (factors down
// to about 1e-35 and up to 6e34): two exponentials and four products per element.
// Otherwise (down to lower_bound -10) the operands are referenced to the chunk's token
// 7, which keeps every factor within e^{8 |lb|}: K_b = k e^{G - Gref}, Q_b likewise, and
// the consumers scale their bf16 copy of the state by e^{Gref} per key channel. Either
// way K_b, Q_b and K_inv = k e^{r - G} are both the consumers' operands and stage B's
// for R and A^qk.
template <typename TSt, bool SG, bool SEG, bool CSR>
__global__ __launch_bounds__(f_threads<SEG>()) void kf_fused(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ graw, const uint16_t *__restrict__ braw, const TSt *s0, TSt *s1,
    uint16_t *__restrict__ out, const int32_t *__restrict__ tok_off, const int32_t *__restrict__ chunk_off, int H,
    float lb, float scale, const int32_t *__restrict__ seg_off, int N, int seg_len, int seg_first,
    float *__restrict__ sfin,
    uint16_t *__restrict__ phi, uint16_t *__restrict__ ybuf, const int32_t *__restrict__ order)
{
    constexpr int kPBytes = slot_bytes<CSR>();
    constexpr int NP = kFPrep, AW = kAW, NE = kNE;
    __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<CSR>()];
    char *const slots = lds;
    char *const inring = lds + kFSlots * kPBytes;
    char *const parts = inring + NP * kFIn * kIBytes;

    // the wave index is uniform over the wave: keep it scalar so role branches and
    // the address arithmetic built on it stay in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.x % H;
    int n, nch, tb, seg = 0, gseg = 0, cs = 0;  // cs: the segment's first chunk in its sequence
    if constexpr (SEG) {
        seg = blockIdx.x / H;
        if (seg >= seg_off[N]) return;  // past the last segment: uniform, before any barrier
        n = find_seq(seg_off, N, seg);
        gseg = seg - seg_off[n];
        cs = seg_start(gseg, seg_len, seg_first);
        nch = min(gseg == 0 ? seg_first : seg_len, chunk_off[n + 1] - chunk_off[n] - cs);
        tb = tok_off[n] + cs * kC;
    } else {
        n = order[blockIdx.x / H];  // longest sequences first
        nch = chunk_off[n + 1] - chunk_off[n];
        tb = tok_off[n];
    }
    const int te = tok_off[n + 1];
    const int ticks = nch > 0 ? nch + 3 : 0;

    // stage-B waves after the stage-A waves: the inverse of even chunks, role 1 (A^qk and
    // beta), and the inverse of odd chunks (the last wave, after the transfer-run waves in
    // the segmented form), on SIMDs 0, 1 and 2
    constexpr int w_inv_odd = kFCons + NP + 2 + (SEG ? kFCons : 0);
    const bool stage_b = w == kFCons + NP || w == kFCons + NP + 1 || w == w_inv_odd;
    if (stage_b) {
        // ================================================================ stage-B waves
        if (nch == 0) return;  // uniform over the workgroup: no barrier is entered
        const int role = w == kFCons + NP + 1 ? 1 : 0;
        const int parity = w == w_inv_odd ? 1 : 0;  // inverse waves: chunks of this parity
        const int tok = lane & 15, g = lane >> 4;  // D layout: rows 4g+r, column tok
        // A B^T over the 128 key channels of the slot's K_b, Q_b and K_inv blocks (32-channel
        // slices in the consumers' lane order): one chained 16x16x32 product per slice (fp32
        // accumulation). Both operands carry the same channel permutation, so the sum runs
        // over the key channels as such.
        const int ls = swz(lane);
        auto contract = [&](const char *P, int offa, int offb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
                acc = mma32(reinterpret_cast<const bf16x8 *>(P + mm * 1024 + offa)[ls],
                            reinterpret_cast<const bf16x8 *>(P + mm * 1024 + offb)[ls], acc);
            return acc;
        };
        bar_sync();  // start: the stage-A waves have waited for chunk 0 in their rings
        if (role == 0) {
            // (A^kk)^T = (I + M)^-1 with M = R^T (strictly upper triangular), by block
            // inversion over four levels of diagonal blocks (2, 4, 8, 16 rows): with X
            // the inverse of the diagonal blocks of one level and C the part of M in the
            // off-diagonal blocks of the next, X - X C X inverts the next level's blocks
            // ([[A, B], [0, D]]^-1 = [[A^-1, -A^-1 B D^-1], [0, D^-1]]). Every value formed
            // is a block of the inverse or a sum of eight bounded products, so the fp16
            // operands (fp32 accumulation) lose nothing to cancellation. The doubling
            // product (I - M)(I + M^2)(I + M^4)(I + M^8) takes as many products but forms
            // M^8, whose entries reach the thousands when the keys of a chunk are
            // correlated and barely decay; they then cancel, and fp16 operands leave
            // errors of order one. Each chunk c of this wave's parity takes two ticks: the
            // first half at tick c+1, the second at tick c+2. One loop iteration covers
            // both, so the values carried between them stay in the same registers.
            int tau = 0;
#pragma unroll 1
            for (; tau <= parity; ++tau) tick_sync();  // ticks before chunk parity's first half
#pragma unroll 1
            for (int c = parity; c < nch; c += 2, tau += 2) {
                const char *X = parts + (c & 1) * kXBytes;
                char *P = slots + (c % kFSlots) * kPBytes;
                // first half (tick c + 1): R, R^T and the first levels of the inverse
                const f32x4 Rs = contract(P, kPKB, kPKI), RTs = contract(P, kPKI, kPKB);
                const f32x4 beta_a = *reinterpret_cast<const f32x4 *>(X + kXBeta + 16 * g);
                const float beta_b = reinterpret_cast<const float *>(X + kXBeta)[tok];
                // rk = 1 / |k| per token, formed by consumer wave 3 in tick c
                const float rkb = reinterpret_cast<const float *>(P + kPSC)[tok];
                const f32x4 rka = *reinterpret_cast<const f32x4 *>(P + kPSC + 16 * g);
                // D layout: element r is row a = 4g + r, column tok. R holds R (lower), RT
                // holds R^T = M; blk(L, x) keeps the part of x in level L's off-diagonal
                // blocks (same block of 2^L rows and columns, different half)
                f32x4 R, RT;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = 4 * g + r;
                    R[r] = (tok < a) ? beta_a[r] * rka[r] * rkb * Rs[r] : 0.f;
                    RT[r] = (a < tok) ? beta_b * rkb * rka[r] * RTs[r] : 0.f;
                }
                auto blk = [&](int L, f32x4 x) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int a = 4 * g + r;
                        x[r] = ((a >> L) == (tok >> L) && (a >> (L - 1)) != (tok >> (L - 1))) ? x[r] : 0.f;
                    }
                    return x;
                };
                // level 1: Xi = I - C_1 (2 x 2 blocks), XiT = Xi^T = I - C_1^T
                f32x4 Xi = eye_plus(blk(1, RT), -1.f, g, tok), XiT = eye_plus(blk(1, R), -1.f, g, tok);
                // level 2: Y = C_2 Xi; Xi <- Xi - Xi Y, XiT <- XiT - Y^T XiT
                {
                    const f32x4 Y = mm16_h(blk(2, R), Xi);
                    const f32x4 Z = mm16_h(XiT, Y), ZT = mm16_h(Y, XiT);
                    Xi -= Z;
                    XiT -= ZT;
                }
                const f32x4 Y3 = mm16_h(blk(3, R), Xi);  // level 3's Y (its update of Xi next tick)
                tick_sync();
                // second half (tick c + 2): level 3's update, level 4 (Xi only), the store
                {
                    const f32x4 Z = mm16_h(XiT, Y3), ZT = mm16_h(Y3, XiT);
                    Xi -= Z;
                    XiT -= ZT;
                }
                const f32x4 AT = Xi - mm16_h(XiT, mm16_h(blk(4, R), Xi));  // (A^kk)^T in D layout
                f32x4 ABT;  // rk_b beta_a A^kk[b][a]: E' = Diag(rk) A^kk Diag(beta) Ebar
#pragma unroll
                for (int r = 0; r < 4; ++r) ABT[r] = rkb * beta_a[r] * AT[r];
                reinterpret_cast<bf16x8 *>(P + kPAB)[lane] = split8(ABT);
                tick_sync();
            }
#pragma unroll 1
            for (; tau < ticks; ++tau) tick_sync();  // the rest only keep the barrier count
            return;
        }
#pragma unroll 1
        for (int tau = 0; tau < ticks; ++tau) {
            if (tau >= 1 && tau - 1 < nch) {
                const int c = tau - 1;
                char *P = slots + (c % kFSlots) * kPBytes;
                const f32x4 AQs = contract(P, kPKI, kPQB);
                const float rqb = reinterpret_cast<const float *>(P + kPSC + 64)[tok];  // s rq
                f32x4 AQT;  // chi_{b,a} / rk_a = s rq_b (q_b . k_a decayed), a <= b
#pragma unroll
                for (int r = 0; r < 4; ++r) AQT[r] = (4 * g + r <= tok) ? rqb * AQs[r] : 0.f;
                reinterpret_cast<bf16x8 *>(P + kPAQ)[lane] = split8(AQT);
            }
            if (tau < nch && lane < 16) {
                // beta of chunk c = tau from the raw beta_raw in stage-A wave 0's ring (landed
                // before the last barrier, refilled only next tick): the low or high half of
                // the aligned dword; rows past the end of the sequence get beta = 0 (absent)
                const int c = tau, t = lane;
                const int t0 = tb + c * kC;
                const int brow = min(t0 + t, te - 1);
                const int64_t eo = ((int64_t)brow * H + h) * 2;
                const bool bhi = (reinterpret_cast<uintptr_t>(reinterpret_cast<const char *>(braw) + eo) & 2) != 0;
                const uint32_t bw = *reinterpret_cast<const uint32_t *>(inring + (c % kFIn) * kIBytes + kIB + t * 4);
                const float beta = (t0 + t < te) ? sigmoid_fast(bhi ? bf_hi(bw) : bf_lo(bw)) : 0.f;
                reinterpret_cast<float *>(parts + (c & 1) * kXBytes + kXBeta)[t] = beta;
            }
            tick_sync();
        }
        return;
    }
    if (w >= kFCons && w < kFCons + NP) {
        // ================================================================ stage-A waves
        if (nch == 0) return;  // uniform over the workgroup: no barrier is entered
        const int m = w - kFCons;
        const int t = lane & 15, sg = lane >> 4;  // token; channel subgroup of NE
        const int cl0 = AW * m + NE * sg;         // the lane's first key channel
        char *const myin = inring + m * kFIn * kIBytes;
        const char *const qb8 = reinterpret_cast<const char *>(q);
        const char *const kb8 = reinterpret_cast<const char *>(k);
        const char *const gb8 = reinterpret_cast<const char *>(graw);
        const char *const vb8 = reinterpret_cast<const char *>(v);
        const char *const bb8 = reinterpret_cast<const char *>(braw);

        // this wave's 32-channel slices of chunk c into input slot `slot` (a load's lane l
        // writes LDS bytes 16 l on from its base)
        auto dma_chunk = [&](int c, int slot) {
            c = min(c, nch - 1);  // past the end: re-read the last chunk (never consumed)
            char *dst = myin + slot * kIBytes;
            // the dword holding beta_raw[brow][h] (and a scalar g_raw[brow][h]): rounding
            // the address down to 4 bytes stays inside the 4-byte word, hence inside the
            // page, that holds the element
            const int brow = min(tb + c * kC + (lane & 15), te - 1);
            const int64_t eo = ((int64_t)brow * H + h) * 2;
            // one load per array: lane = (row l/4, 16-byte piece l%4)
            const int row = min(tb + c * kC + (lane >> 2), te - 1);
            const int64_t off = (((int64_t)row * H + h) * kD + AW * m) * 2 + (lane & 3) * 16;
            __builtin_amdgcn_global_load_lds(qb8 + off, (lds_void *)(dst + kIQ), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(kb8 + off, (lds_void *)(dst + kIK), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb8 + off, (lds_void *)(dst + kIV), 16, 0, 0);
            if constexpr (!SG) __builtin_amdgcn_global_load_lds(gb8 + off, (lds_void *)(dst + kIG), 16, 0, 0);
            if (lane < kC) {  // one dword per token, lanes 0-15 (64 bytes of the slot)
                if constexpr (SG) {
                    const uintptr_t ga = reinterpret_cast<uintptr_t>(gb8 + eo);
                    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(ga & ~(uintptr_t)3),
                                                     (lds_void *)(dst + kIG), 4, 0, 0);
                }
                const uintptr_t ba = reinterpret_cast<uintptr_t>(bb8 + eo);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(ba & ~(uintptr_t)3),
                                                 (lds_void *)(dst + kIB), 4, 0, 0);
            }
        };
#pragma unroll
        for (int i = 0; i < kFIn - 1; ++i) dma_chunk(i, i);
        // The inputs of chunk c are read from LDS into registers at the end of tick
        // c - 1 (chunk 0: here), so their LDS latency overlaps the other waves' work.
        typedef uint32_t uNE __attribute__((ext_vector_type(NE / 2)));
        uNE qa, ka, ga, va;
        auto read_inputs = [&](int c) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kFPending) : "memory");  // chunk c landed
            const char *I = myin + (c % kFIn) * kIBytes + t * (2 * AW) + sg * (2 * NE);
            qa = *reinterpret_cast<const uNE *>(I + kIQ);
            ka = *reinterpret_cast<const uNE *>(I + kIK);
            if constexpr (SG) {
                ga[0] = *reinterpret_cast<const uint32_t *>(myin + (c % kFIn) * kIBytes + kIG + t * 4);
            } else {
                ga = *reinterpret_cast<const uNE *>(I + kIG);
            }
            va = *reinterpret_cast<const uNE *>(I + kIV);
        };
        read_inputs(0);
        tick_sync();  // start: chunk 0 has landed in this wave's ring (stage B reads every ring)

        const float lb2 = lb * kLog2e;
        // one tick of stage A on chunk c. The prepared slot c % kFSlots is a compile-time
        // constant (the loop below steps through the slots in turn), so the slot's LDS
        // addresses fold into instruction offsets instead of being rebuilt every tick.
        auto stage_a = [&](const int c, auto slot_tag) {
            constexpr int slot = decltype(slot_tag)::value;
            // chunk c - 1's slot is free (its inputs were read before the last barrier,
            // by this wave and by stage B): refill it with chunk c + kFIn - 1
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            dma_chunk(c + kFIn - 1, (c + kFIn - 1) % kFIn);
            const int t0 = tb + c * kC, len = min(kC, te - t0);
            // rows past the end of the sequence hold copies of its last row; zero
            // gate and beta make them absent: they reach only the masked triangles
            // of R and A^qk, rows of E' that come out exactly zero, and output rows
            // that are never stored
            const bool valid = t < len;

            // gate in log2 units: lb2 sigma(x) = 1 / ((1 + e^-x) / lb2), one fma and one
            // reciprocal after the exponential. Rows past the end (and lower_bound 0) take
            // -FLT_MAX for 1/lb2: their gate is -0 or a denormal, which decays by nothing
            // (a finite stand-in, so e^-x = 0 from x = +inf meets no 0 * inf)
            const float ilb = (valid && lb2 != 0.f) ? 1.f / lb2 : -3.402823466e38f;
            auto gate2 = [&](float x) {
                return __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(-x * kLog2e), ilb, ilb));
            };
            float qf[NE], kf[NE], gf[NE];
#pragma unroll
            for (int e = 0; e < NE / 2; ++e) {
                qf[2 * e] = bf_lo(qa[e]);
                qf[2 * e + 1] = bf_hi(qa[e]);
                kf[2 * e] = bf_lo(ka[e]);
                kf[2 * e + 1] = bf_hi(ka[e]);
            }
            if constexpr (SG) {  // one gate and one prefix sum serve every channel
                const int grow = min(t0 + t, te - 1);
                const int64_t eo = ((int64_t)grow * H + h) * 2;  // byte offset of [grow][h]
                const bool ghi = (reinterpret_cast<uintptr_t>(gb8 + eo) & 2) != 0;
                float x = gate2(ghi ? bf_hi(ga[0]) : bf_lo(ga[0]));
                // rounded exactly as the per-channel gate below, step by step
                asm("" : "+v"(x));
                x += row_shr<1>(x);
                x += row_shr<2>(x);
                x += row_shr<4>(x);
                x += row_shr<8>(x);
                asm("" : "+v"(x));
#pragma unroll
                for (int i = 0; i < NE; ++i) gf[i] = x;
            } else {
#pragma unroll
                for (int e = 0; e < NE / 2; ++e) {
                    gf[2 * e] = bf_lo(ga[e]);
                    gf[2 * e + 1] = bf_hi(ga[e]);
                }
                // gate (log2 units) and prefix sum over tokens, one shift step at a time over
                // all channels, so consecutive DPP adds touch different registers; the empty
                // asm statements keep each value as computed, so each shifted add stays a
                // single DPP add
#pragma unroll
                for (int i = 0; i < NE; ++i) {
                    gf[i] = gate2(gf[i]);
                    asm("" : "+v"(gf[i]));
                }
#pragma unroll
                for (int i = 0; i < NE; ++i) gf[i] += row_shr<1>(gf[i]);
#pragma unroll
                for (int i = 0; i < NE; ++i) gf[i] += row_shr<2>(gf[i]);
#pragma unroll
                for (int i = 0; i < NE; ++i) gf[i] += row_shr<4>(gf[i]);
#pragma unroll
                for (int i = 0; i < NE; ++i) {
                    gf[i] += row_shr<8>(gf[i]);
                    asm("" : "+v"(gf[i]));
                }
            }
            char *P = slots + slot * kPBytes;
            // per element: K_b = k e^{G - r}, Q_b = q e^{G - r}, K_inv = k e^{r - G} and
            // K_end = K_inv e^{G_last - r} (the factor from token 15's lane of the row);
            // gamma = e^{G_last}, and e^{r} for the consumers when r is token 7's G
            float ke[NE], gam[NE], er[NE];
            bf16x4 kb4[NE / 4], qb4[NE / 4], ki4[NE / 4];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                float up, dn, cl;
                if constexpr (CSR) {  // r = 0
                    up = __builtin_amdgcn_exp2f(gf[i]);
                    dn = __builtin_amdgcn_exp2f(-gf[i]);
                    cl = row_bcast<15>(up);
                    gam[i] = up;
                } else {  // r = G of token 7: every factor within e^{8 |lb|}
                    const float gref = row_bcast<7>(gf[i]), d = gf[i] - gref;
                    up = __builtin_amdgcn_exp2f(d);
                    dn = __builtin_amdgcn_exp2f(-d);
                    cl = row_bcast<15>(up);
                    er[i] = __builtin_amdgcn_exp2f(gref);
                    gam[i] = cl * er[i];
                }
                const float ki = kf[i] * dn;
                kb4[i >> 2][i & 3] = (__bf16)(kf[i] * up);
                qb4[i >> 2][i & 3] = (__bf16)(qf[i] * up);
                ki4[i >> 2][i & 3] = (__bf16)ki;
                ke[i] = ki * cl;
            }
            // raw K_end as a bf16 hi/lo pair: channel cr = AW m + NE sg + i sits in tile pair
            // cr / 32, consumer lane (cr % 16) + 16 (t / 4), tile half (cr / 16) % 2, element
            // t % 4 (hi part; lo 8 bytes on); rounded in pairs, stored as halves
#pragma unroll
            for (int i = 0; i < NE; i += 2) {
                const uint32_t ph = pk_bf16(f32x2{ke[i], ke[i + 1]});
                const uint32_t pl = pk_bf16(f32x2{ke[i] - bf_lo(ph), ke[i + 1] - bf_hi(ph)});
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int cr = cl0 + i + j, kc = cr & 15, hf = (cr >> 4) & 1;
                    char *d = P + kPKE + (cr >> 5) * 2048 + swz(kc + 16 * (t >> 2)) * 32 + hf * 16 + (t & 3) * 2;
                    *reinterpret_cast<uint16_t *>(d) = (uint16_t)(ph >> (16 * j));
                    *reinterpret_cast<uint16_t *>(d + 8) = (uint16_t)(pl >> (16 * j));
                }
            }
            // K_b, Q_b and K_inv in the consumer's 16x16x32 A order: the 4 channels from cb
            // sit in tile pair cb / 32, consumer lane t + 16 gd, elements e0 .. e0 + 3
#pragma unroll
            for (int j = 0; j < NE / 4; ++j) {
                const int cb = cl0 + 4 * j, q4 = (cb & 31) >> 2;
                const int gd = q4 & 3, e0 = (q4 >> 2) * 4;
                const int o = (cb >> 5) * 1024 + swz(t + 16 * gd) * 16 + e0 * 2;
                *reinterpret_cast<bf16x4 *>(P + kPKB + o) = kb4[j];
                *reinterpret_cast<bf16x4 *>(P + kPQB + o) = qb4[j];
                *reinterpret_cast<bf16x4 *>(P + kPKI + o) = ki4[j];
            }
            if (t == 15) {  // gamma (and e^{r}) per key channel
#pragma unroll
                for (int j = 0; j < NE / 4; ++j) {
                    float *gm = reinterpret_cast<float *>(P + kPGM) + cl0 + 4 * j;
                    *reinterpret_cast<f32x4 *>(gm) = f32x4{gam[4 * j], gam[4 * j + 1], gam[4 * j + 2], gam[4 * j + 3]};
                    if constexpr (!CSR) {
                        float *e = reinterpret_cast<float *>(P + kPER) + cl0 + 4 * j;
                        *reinterpret_cast<f32x4 *>(e) = f32x4{er[4 * j], er[4 * j + 1], er[4 * j + 2], er[4 * j + 3]};
                    }
                }
            }
            *reinterpret_cast<uNE *>(P + kPV + t * kVRow + cl0 * 2) = valid ? va : uNE{};
            if (c + 1 < nch) read_inputs(c + 1);
        };
        // ticks past the last chunk only keep the barrier count
#pragma unroll 1
        for (int tau = 0; tau < ticks; tau += kFSlots) {
            if (tau < nch) stage_a(tau, std::integral_constant<int, 0>{});
            tick_sync();
            if (tau + 1 < ticks) {
                if (tau + 1 < nch) stage_a(tau + 1, std::integral_constant<int, 1>{});
                tick_sync();
            }
            if (tau + 2 < ticks) {
                if (tau + 2 < nch) stage_a(tau + 2, std::integral_constant<int, 2>{});
                tick_sync();
            }
            if (tau + 3 < ticks) {
                if (tau + 3 < nch) stage_a(tau + 3, std::integral_constant<int, 3>{});
                tick_sync();
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // nothing still landing in LDS at exit
        return;
    }

    // ==================================================================== consumers
    // Lane (col, g) of consumer wave cw holds, for column tile u, rows 4g..4g+3 of
    // the 16x16 state tiles st[u][t] = S^T[16t .., 32cw + 16u + col] (D layout).
    // MODE 0: the whole sequence; MODE 1: a segment's run from S = 0 (segment 0: the
    // initial state); MODE 2: a segment's transfer run, from S = I with v = 0.
    auto consume = [&](auto mode_tag, const int cw) {
    constexpr int MODE = decltype(mode_tag)::value;
    const int g = lane >> 4, col = lane & 15, sl = swz(lane);
    const int64_t sbase = (((int64_t)n * H + h) * kD + 32 * cw + col) * kD + 4 * g;
    f32x4 st[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (MODE == 2) {  // identity: S^T[16t + 4g + r][32cw + 16u + col]
#pragma unroll
                for (int r = 0; r < 4; ++r) st[u][t][r] = (16 * t + 4 * g + r == 32 * cw + 16 * u + col) ? 1.f : 0.f;
            } else {
                st[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    if (MODE != 2 && s0 != nullptr && gseg == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t) st[u][t] = ld_state4(s0 + sbase + (int64_t)16 * kD * u + 16 * t);
    }
    if (ticks > 0) bar_sync();  // start: the stage-A waves have waited for chunk 0 in their rings
#pragma unroll 1
    for (int tau = 0; tau < ticks; ++tau) {
        if (MODE != 2 && tau < nch && (cw & 1)) {
            // per-token scales of chunk tau from the raw inputs in the stage-A rings
            // (landed before the last barrier, refilled only next tick). The squared
            // norms of the 16 k rows (wave 3) or q rows (wave 1) are the diagonal of their
            // Gram matrix: four 16x16x32 bf16 products over the 128 channels, exact
            // products accumulated in fp32, with the same registers as both operands.
            // Lane (token i, group i/4) holds |x_i|^2. rk = 1/|k| and s rq = s/|q| go to
            // the chunk's slot for stage B (next tick) and for the consumers' own step
            // three ticks later. Waves 1 and 3 share their SIMDs with the lighter stage-B
            // roles.
            static_assert(kFCons == 4, "consumer waves 1 and 3 form the norms");
            const bool isk = cw == 3;
            const char *I = inring + (tau % kFIn) * kIBytes + col * 64 + g * 16 + (isk ? kIK : kIQ);
            f32x4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 x = *reinterpret_cast<const bf16x8 *>(I + ks * kFIn * kIBytes);
                gram = mma32(x, x, gram);
            }
            if ((col >> 2) == g) {
                const float n2 = (col & 2) ? ((col & 1) ? gram[3] : gram[2]) : ((col & 1) ? gram[1] : gram[0]);
                float *sc = reinterpret_cast<float *>(slots + (tau % kFSlots) * kPBytes + kPSC);
                const float r = __builtin_amdgcn_rsqf(n2 + kL2Eps);
                sc[isk ? col : 16 + col] = isk ? r : scale * r;
            }
        }
        if (tau >= 3) {
            const int c = tau - 3;
            const char *L = slots + (c % kFSlots) * kPBytes;
            const int t0 = tb + c * kC, len = min(kC, te - t0);
            // K_b S^T and Q_b S^T for both column tiles (bf16 state operand; with token 7's
            // reference r, the state scaled by e^{r} per key channel: K_b e^{r} = k e^G).
            // K_b and Q_b are read here, in the tick that uses them. Loading them into
            // registers before the previous barrier gave wrong outputs with ROCm 7.2.0's
            // hipcc (AMD clang 22, roc-7.2.0): the code it generated wrote a VALU result
            // into an accumulator operand of an MFMA still in flight.
            f32x4 xk[2], xq[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) xk[u] = xq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(L + kPKB + p * 1024 + sl * 16);
                const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(L + kPQB + p * 1024 + sl * 16);
                f32x4 er0 = {1.f, 1.f, 1.f, 1.f}, er1 = er0;
                if constexpr (!CSR) {
                    er0 = *reinterpret_cast<const f32x4 *>(L + kPER + (32 * p + 4 * g) * 4);
                    er1 = *reinterpret_cast<const f32x4 *>(L + kPER + (32 * p + 16 + 4 * g) * 4);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf16x8 sb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sb[r] = (__bf16)(CSR ? st[u][2 * p][r] : st[u][2 * p][r] * er0[r]);
                        sb[4 + r] = (__bf16)(CSR ? st[u][2 * p + 1][r] : st[u][2 * p + 1][r] * er1[r]);
                    }
                    xk[u] = mma32(kb, sb, xk[u]);
                    // operands swapped: (Q_b S^T)^T, lane (token, g) holds value channels 4g..4g+3
                    xq[u] = mma32(sb, qb, xq[u]);
                }
            }
            const f32x4 rk4 = *reinterpret_cast<const f32x4 *>(L + kPSC + 16 * g);
            const float rq1 = reinterpret_cast<const float *>(L + kPSC + 64)[col];
            const bf16x8 ab = *reinterpret_cast<const bf16x8 *>(L + kPAB + lane * 16);
            const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(L + kPAQ + lane * 16);
            const bf16x4 ab_h = {ab[0], ab[1], ab[2], ab[3]}, ab_l = {ab[4], ab[5], ab[6], ab[7]};
            const bf16x4 aq_h = {aq[0], aq[1], aq[2], aq[3]}, aq_l = {aq[4], aq[5], aq[6], aq[7]};
            bf16x4 eh[2], el[2];
            // output row of this lane's token: value channels 32w + 16u + 4g .. +3 of tile u
            uint16_t *orow = out + ((int64_t)(t0 + col) * H + h) * kD + 32 * cw + 4 * g;
            u32x4 yv;  // MODE 2: y of this lane's token, both column tiles
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int vcol = 32 * cw + 16 * u + col;
                f32x4 eb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (MODE == 2) {
                        eb[r] = -rk4[r] * xk[u][r];
                    } else {
                        const uint16_t vr =
                            *reinterpret_cast<const uint16_t *>(L + kPV + (4 * g + r) * kVRow + vcol * 2);
                        eb[r] = bf16_bits_to_f32(vr) - rk4[r] * xk[u][r];  // rows past the end hold zeros
                    }
                    xq[u][r] *= rq1;
                }
                // E' = Diag(rk) E with split-bf16 operands: A_h eb_h + A_l eb_h + A_h eb_l (an
                // fp32 16x16x4 form measured slower: its four chained products sit on the
                // recurrence's critical path)
                bf16x4 eb_h, eb_l, e_h, e_l;
                split4t_packed(eb, eb_h, eb_l);
                f32x4 E = {0.f, 0.f, 0.f, 0.f};
                E = mma16(ab_h, eb_h, E);
                E = mma16(ab_l, eb_h, E);
                E = mma16(ab_h, eb_l, E);
                split4t_packed(E, e_h, e_l);
                eh[u] = e_h;
                el[u] = e_l;
                // O^T = (Q_b S^T)^T Diag(rq) + E'^T (A^qk / Diag(rk))^T: the D-layout E tiles are
                // the A operand of the transposed product, the stored A^qk block its B operand
                f32x4 O = mma16(e_h, aq_h, xq[u]);
                O = mma16(e_h, aq_l, O);
                O = mma16(e_l, aq_h, O);
                const u32x2 ob = {pk_bf16(f32x2{O[0], O[1]}), pk_bf16(f32x2{O[2], O[3]})};
                if constexpr (MODE == 2) {
                    yv[2 * u] = ob[0];
                    yv[2 * u + 1] = ob[1];
                } else if (col < len) {
                    *reinterpret_cast<u32x2 *>(orow + 16 * u) = ob;
                }
            }
            if constexpr (MODE == 2) {
                // the chunk's y tile: k step cw of the correction's operand, lane (token col,
                // group g) holding channels 32 cw + 4 g + (0..3) and 32 cw + 16 + 4 g + (0..3);
                // rows past the end are stored too and never used
                const int64_t tile = (int64_t)(chunk_off[n] + cs + c) * H + h;
                *reinterpret_cast<u32x4 *>(ybuf + (tile * kFCons + cw) * (64 * 8) + lane * 8) = yv;
            }
            // S^T <- Diag(gamma) S^T + K_end^T E', K_end = hi + lo and E' = eh + el:
            // [hi | lo] against [eh; eh] in one 16x16x32 product, then hi against el in a
            // 16x16x16 one. Such a pair needs about five wait states between its products
            // (see mma16); here the two column tiles' products interleave, which puts three
            // or more independent products between them, and a host test checks the
            // generated code for it. A second 16x16x32 product instead costs 3% at C3.
            bf16x8 ehh[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) ehh[u] = cat8(eh[u], eh[u]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(L + kPKE + (t >> 1) * 2048 + sl * 32 + (t & 1) * 16);
                const bf16x4 kt = {k8[0], k8[1], k8[2], k8[3]};
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(L + kPGM + (16 * t + 4 * g) * 4);
#pragma unroll
                for (int u = 0; u < 2; ++u) st[u][t] = mma16(kt, el[u], mma32(k8, ehh[u], st[u][t] * gm));
            }
        }
        // waves 1 and 3 stored the chunk's per-token scales above, which stage B reads
        // next tick: complete them before the barrier (every value read is used already)
        tick_sync();
    }
    if constexpr (MODE == 0) {
        if (s1) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < 8; ++t) st_state4(s1 + sbase + (int64_t)16 * kD * u + 16 * t, st[u][t]);
        }
    } else if constexpr (MODE == 1) {
        // tile order: st[u][t] holds keys 16t + 4g .. +3 of value row 32 cw + 16 u + col
        float *const F = sfin + ((int64_t)seg * H + h) * (kD * kD);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                *reinterpret_cast<f32x4 *>(F + state_tile(32 * cw + 16 * u + col, 16 * t + 4 * g)) = st[u][t];
    } else {
        // Phi^T as the scan's matrix-core A operand, split into bf16 hi and lo: per
        // (segment, head), key tile t and k step cw, 512 hi values then 512 lo ones; lane
        // 16 (2u + col/8) + 4g + r of tile t holds channels 32 cw + 16 u + 8 (col/8) + 0..7
        // of key 16t + 4g + r, this lane's value at element col % 8
        uint16_t *const P = phi + ((int64_t)seg * H + h) * (2 * kD * kD) + cw * (2 * 512) + (col & 7);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                bf16x4 hi, lo;
                split4t(st[u][t], hi, lo);
                // whole vectors reinterpreted, then indexed: a bit cast of one element
                // of a bf16 vector compiled to element 0 for every index (ROCm 7.2.0)
                const i16x4 hb = __builtin_bit_cast(i16x4, hi), lb = __builtin_bit_cast(i16x4, lo);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint16_t *d = P + t * (4 * 2 * 512) + (16 * (2 * u + (col >> 3)) + 4 * g + r) * 8;
                    d[0] = (uint16_t)hb[r];
                    d[512] = (uint16_t)lb[r];
                }
            }
    }
    };
    if constexpr (SEG) {
        if (w < kFCons) {
            consume(std::integral_constant<int, 1>{}, w);
        } else if (nch > 0) {  // transfer-run waves
            if (gseg > 0) {
                consume(std::integral_constant<int, 2>{}, w - (kFCons + NP + 2));
            } else {
#pragma unroll 1
                for (int tau = 0; tau <= ticks; ++tau) bar_sync();  // the start barrier and every tick's
            }
        }
    } else {
        consume(std::integral_constant<int, 0>{}, w);
    }
}

template <typename TSt, bool SG, bool SEG, bool CSR>
static hipError_t launch_fused_t(const Problem &p, hipStream_t s)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    const int32_t *seg = SEG ? reinterpret_cast<const int32_t *>(p.ws + p.lay.seg_off) : nullptr;
    float *sfin = SEG ? reinterpret_cast<float *>(p.ws + p.lay.sfin) : nullptr;
    uint16_t *phi = SEG ? reinterpret_cast<uint16_t *>(p.ws + p.lay.phi) : nullptr;
    uint16_t *ybuf = SEG ? reinterpret_cast<uint16_t *>(p.ws + p.lay.ybuf) : nullptr;
    const int64_t groups = (SEG ? p.lay.seg_max : p.N) * p.H;
    hipLaunchKernelGGL((kf_fused<TSt, SG, SEG, CSR>), dim3((unsigned)groups), dim3(f_threads<SEG>()), 0, s,
                       (const uint16_t *)p.q, (const uint16_t *)p.k, (const uint16_t *)p.v, (const uint16_t *)p.g,
                       (const uint16_t *)p.beta, (const TSt *)p.s0, (TSt *)p.s1, (uint16_t *)p.out, tok, chk, p.H,
                       p.lb, p.scale, seg, (int)p.N, (int)p.lay.seg_len, (int)p.lay.seg_first, sfin, phi, ybuf,
                       SEG ? nullptr : reinterpret_cast<const int32_t *>(p.ws + p.lay.order));
    return hipGetLastError();
}

// decays referenced to the chunk start from lower_bound -5 up (see kf_fused)
constexpr float kCsrMinLowerBound = -5.0f;

template <bool SEG, bool CSR>
static hipError_t launch_fused_ref(const Problem &p, hipStream_t s)
{
    if (p.scalar_gate)
        return p.st_bf16 ? launch_fused_t<uint16_t, true, SEG, CSR>(p, s) : launch_fused_t<float, true, SEG, CSR>(p, s);
    return p.st_bf16 ? launch_fused_t<uint16_t, false, SEG, CSR>(p, s) : launch_fused_t<float, false, SEG, CSR>(p, s);
}

template <bool SEG>
static hipError_t launch_fused_any(const Problem &p, hipStream_t s)
{
    return p.lb >= kCsrMinLowerBound ? launch_fused_ref<SEG, true>(p, s) : launch_fused_ref<SEG, false>(p, s);
}

bool fits_fused(const Problem &p, bool seg)
{
    return seg ? grid_fits(p.lay.seg_max * p.H, 1, f_threads<true>()) : grid_fits(p.N * p.H, 1, f_threads<false>());
}

hipError_t launch_fused(const Problem &p, hipStream_t s) { return launch_fused_any<false>(p, s); }
hipError_t launch_fused_seg(const Problem &p, hipStream_t s) { return launch_fused_any<true>(p, s); }

}  // namespace kda
