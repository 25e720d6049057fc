// kda_seg.hip -- the two kernels that finish the segmented single pass.
//
// The segmented pass (kf_fused with SEG, kda_fused.hip) cuts every sequence into
// segments and runs each segment from a zero state (segment 0: the initial
// state), giving its outputs o0, its final state S0 and, from a second run with
// state I and v = 0, its key-space transfer Phi and the vectors y_t = Phi_t (s qhat_t).
// The state recurrence of the Doubleword page "You Could Have Come Up with Kimi
// Delta Attention" (section 4) is linear in (S, v) for fixed q, k, alpha and beta,
// and its transition is the product form of section 4.1, so with S_in the true
// state entering segment g:
//   S at token t = S_in Phi_t + S0_t,      o_t = o0_t + S_in y_t,
//   S_in(g+1) = S_in(g) Phi_g + S0_g,      S_in(0) = initial state.
// kseg_scan walks that chain over the segments of each (sequence, head) with fp32
// matrix-core products; kseg_correct adds S_in y_t to the outputs of every
// segment after the first.
#include "kda_mfma_common.h"

namespace kda {

constexpr int kScanRows = 16;   // value rows per scan workgroup
constexpr int kScanLd = kD + 4;  // padded LDS row (floats)

__device__ __forceinline__ f32x4 mma4f(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kScanWaves = 8;    // one 16-column tile of the state rows each
constexpr int kScanDepth = 3;    // segments whose Phi and S0 are in flight ahead of the chain
constexpr int kScanPhiLd = kD + 16;  // padded LDS row of Phi (floats): the four k rows a
                                     // B-operand read touches fall 16 banks apart

// LDS column of state column k: the 32 columns 4i + g (i = 0..31) that one lane group g
// of the 16x16x4 A operand reads are contiguous, so a lane fetches them 16 bytes at a time
__device__ __forceinline__ int scan_col(int k) { return 32 * (k & 3) + (k >> 2); }

// One workgroup (8 waves) per (sequence, head, 16 value rows). The state rows stay
// in LDS; each step forms S Phi_g + S0_g: wave w owns key columns [16w, 16w+16) and
// contracts over the 128 rows of Phi_g in 16x16x4 fp32 steps, with Phi_g and the S0_g
// rows staged through LDS. Their 16-byte loads run kScanDepth segments ahead of the
// chain (ten memory operations per lane and step, well within what the wait counter
// tracks), into register buffers that the unrolled loop addresses statically.
template <typename TSt>
__global__ __launch_bounds__(64 * kScanWaves) void kseg_scan(const TSt *s0, TSt *s1,
                                                             const int32_t *__restrict__ seg_off, int H,
                                                             const float *__restrict__ sfin,
                                                             const float *__restrict__ phi, float *__restrict__ sin)
{
    constexpr int kThreads = 64 * kScanWaves;
    constexpr int kPhiLoads = kD * kD / 4 / kThreads;  // float4 loads of Phi per lane
    static_assert(kPhiLoads * kThreads * 4 == kD * kD && kScanRows * kD == 4 * kThreads,
                  "Phi in whole passes of float4 loads, the S0 rows in one");
    __shared__ __attribute__((aligned(16))) float S[kScanRows][kScanLd];  // columns in scan_col order
    __shared__ __attribute__((aligned(16))) float Ph[kD][kScanPhiLd];
    __shared__ __attribute__((aligned(16))) float Zs[kScanRows][kScanLd];
    const int n = blockIdx.x / H, h = blockIdx.x % H, r0 = blockIdx.y * kScanRows;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
    const int first = seg_off[n], G = seg_off[n + 1] - first;
    const int64_t mat = (int64_t)kD * kD;
    auto seg_off_of = [&](int sg) { return ((int64_t)sg * H + h) * mat; };
    // this lane's 16-byte pieces: Phi element 4 (tid + it kThreads) and S0 row r0 + zr, columns zc..zc+3
    const int zr = tid / (kD / 4), zc = 4 * (tid % (kD / 4));

    // state entering segment 1: segment 0's run started from the initial state
    for (int i = tid; i < kScanRows * kD; i += kThreads) {
        const int r = i / kD, c = i % kD;
        float x;
        if (G > 0)
            x = sfin[seg_off_of(first) + (int64_t)(r0 + r) * kD + c];
        else
            x = s0 ? ld_elem(s0, ((int64_t)n * H + h) * mat + (int64_t)(r0 + r) * kD + c) : 0.f;
        S[r][scan_col(c)] = x;
    }
    f32x4 pb[kScanDepth][kPhiLoads];
    f32x4 z[kScanDepth];
    auto load_step = [&](int gi, f32x4(&pp)[kPhiLoads], f32x4 &zz) {
        const f32x4 *P = reinterpret_cast<const f32x4 *>(phi + seg_off_of(first + gi));
#pragma unroll
        for (int it = 0; it < kPhiLoads; ++it) pp[it] = P[tid + it * kThreads];
        zz = *reinterpret_cast<const f32x4 *>(sfin + seg_off_of(first + gi) + (int64_t)(r0 + zr) * kD + zc);
    };
    // loads past the last segment re-read it (clamped), so every loop iteration issues
    // the same memory operations and the waits before a buffer's use stay exact
    if (G > 1) {
#pragma unroll
        for (int d = 0; d < kScanDepth; ++d) load_step(min(1 + d, G - 1), pb[d], z[d]);
    }
    __syncthreads();
    auto step = [&](int gi, f32x4(&pp)[kPhiLoads], f32x4 &zz) {
        // the previous step's reads of Ph and Zs ended at its barrier
#pragma unroll
        for (int it = 0; it < kPhiLoads; ++it) {
            const int e = 4 * (tid + it * kThreads);
            *reinterpret_cast<f32x4 *>(&Ph[e / kD][e % kD]) = pp[it];
        }
        *reinterpret_cast<f32x4 *>(&Zs[zr][zc]) = zz;
        load_step(min(gi + kScanDepth, G - 1), pp, zz);  // the buffers are free once stored
        __syncthreads();  // Ph, Zs and the previous step's S rows are in place
        {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = S[zr][scan_col(zc + j)];
            *reinterpret_cast<f32x4 *>(sin + seg_off_of(first + gi) + (int64_t)(r0 + zr) * kD + zc) = x;
        }
        f32x4 a[kD / 16];  // A[row col][k = 4 ks + g] for ks = 0..31
#pragma unroll
        for (int q = 0; q < kD / 16; ++q) a[q] = *reinterpret_cast<const f32x4 *>(&S[col][32 * g + 4 * q]);
        float b[kD / 4];  // B[k = 4 ks + g][column 16 w + col]
#pragma unroll
        for (int ks = 0; ks < kD / 4; ++ks) b[ks] = Ph[4 * ks + g][16 * w + col];
        // four independent accumulation chains (k steps 4i + c go to chain c)
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kD / 4; ++ks) acc[ks & 3] = mma4f(a[ks / 4][ks % 4], b[ks], acc[ks & 3]);
        f32x4 zv;
#pragma unroll
        for (int r = 0; r < 4; ++r) zv[r] = Zs[4 * g + r][16 * w + col];
        __syncthreads();  // every wave has read S, Ph and Zs
        const f32x4 sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + zv;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[4 * g + r][scan_col(16 * w + col)] = sum[r];
    };
    static_assert(kScanDepth == 3, "the loop below is unrolled over the buffers");
    int gi = 1;
#pragma unroll 1
    for (; gi + 2 < G; gi += kScanDepth) {
        step(gi, pb[0], z[0]);
        step(gi + 1, pb[1], z[1]);
        step(gi + 2, pb[2], z[2]);
    }
    if (gi < G) step(gi, pb[0], z[0]);
    if (gi + 1 < G) step(gi + 1, pb[1], z[1]);
    __syncthreads();  // the last step's S rows are in place
    if (s1) {
        for (int i = tid; i < kScanRows * kD; i += kThreads)
            st_elem(s1, ((int64_t)n * H + h) * mat + (int64_t)(r0 + i / kD) * kD + i % kD, S[i / kD][scan_col(i % kD)]);
    }
}

constexpr int kCorrWaves = 8;
constexpr int kCorrTok = 32 * kCorrWaves;  // tokens per workgroup
constexpr int kCorrLd = kD + 8;            // padded LDS row (bf16): rows 4 banks apart

// LDS row of value channel r = 32p + 8g + 4u + i: row 16 (2p + u) + 4g + i. Result tiles
// 2p and 2p + 1 then hold channels 32p + 8g + (0..3) and (4..7) in lane group g, so a
// lane reads and writes eight consecutive output channels (16 bytes) at once.
__device__ __forceinline__ int corr_row(int r) { return (r & ~31) + 16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3); }
// LDS column of key channel c = 32 ks + 16 u + 4 g + i: column 32 ks + 8 g + 4 u + i, the
// order in which the single pass stores a y tile (lane group g of k step ks holds
// channels 32 ks + 4 g + (0..3), then 32 ks + 16 + 4 g + (0..3))
__device__ __forceinline__ int corr_col(int c) { return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3); }

// o_t += S_in y_t for every segment after the first. Workgroup (segment, head, j)
// splits S_in once into bf16 hi and lo halves in LDS, then walks the segment's
// token blocks j, j + gridDim.y, ... of 256 tokens: wave w takes 32 tokens (two
// chunks) and forms (S_in y^T) for them as 16x16 tiles (rows: value channels in the
// order corr_row gives, columns: tokens), so each lane ends with eight consecutive
// value channels of one token. The y of a chunk is one 4 KB tile in operand order.
__global__ __launch_bounds__(64 * kCorrWaves) void kseg_correct(uint16_t *__restrict__ out,
                                                                 const uint16_t *__restrict__ ybuf,
                                                                 const float *__restrict__ sin,
                                                                 const int32_t *__restrict__ tok_off,
                                                                 const int32_t *__restrict__ chunk_off,
                                                                 const int32_t *__restrict__ seg_off, int N, int H,
                                                                 int seg_len, int seg_first)
{
    __shared__ __attribute__((aligned(16))) uint16_t Shi[kD][kCorrLd];
    __shared__ __attribute__((aligned(16))) uint16_t Slo[kD][kCorrLd];
    const int seg = blockIdx.x / H, h = blockIdx.x % H;
    if (seg >= seg_off[N]) return;
    const int n = find_seq(seg_off, N, seg), gi = seg - seg_off[n];
    if (gi == 0) return;
    const int tb = tok_off[n] + seg_start(gi, seg_len, seg_first) * kC;  // segments after the first: seg_len chunks
    const int te = min(tok_off[n + 1], tb + seg_len * kC);
    if (tb + (int)blockIdx.y * kCorrTok >= te) return;  // uniform over the workgroup, before any barrier

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
    const float *Sg = sin + ((int64_t)seg * H + h) * kD * kD;
    constexpr int kSplitIt = kD * kD / 4 / (64 * kCorrWaves);
    static_assert(kD * kD / 4 % (64 * kCorrWaves) == 0, "the split covers S_in in whole passes");
    f32x4 sx[kSplitIt];  // every load of the split issued before the first LDS write
#pragma unroll
    for (int it = 0; it < kSplitIt; ++it) sx[it] = reinterpret_cast<const f32x4 *>(Sg)[tid + it * 64 * kCorrWaves];
#pragma unroll
    for (int it = 0; it < kSplitIt; ++it) {
        const int i = tid + it * 64 * kCorrWaves;
        const f32x4 x = sx[it];
        const int r = (4 * i) / kD, c = (4 * i) % kD;
        const u32x4 u = __builtin_bit_cast(u32x4, x);
        // hi truncated (x - hi is exact in fp32), lo the remainder rounded
        const u32x2 hi = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u), __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
        const f32x2 r01 = {x[0] - __uint_as_float(u[0] & 0xffff0000u), x[1] - __uint_as_float(u[1] & 0xffff0000u)};
        const f32x2 r23 = {x[2] - __uint_as_float(u[2] & 0xffff0000u), x[3] - __uint_as_float(u[3] & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(&Shi[corr_row(r)][corr_col(c)]) = hi;
        *reinterpret_cast<u32x2 *>(&Slo[corr_row(r)][corr_col(c)]) = u32x2{pk_bf16(r01), pk_bf16(r23)};
    }
    __syncthreads();

    const int64_t rowst = (int64_t)H * kD;
#pragma unroll 1
    for (int tlo = tb + blockIdx.y * kCorrTok; tlo < te; tlo += gridDim.y * kCorrTok) {
        // every load of the block's two token tiles is issued before any product, so
        // each wave keeps 2 x (512 B y + 256 B o) per lane-row in flight at once
        bf16x8 yb[2][kD / 32];
        u32x4 ov[2][kD / 32];
        bool live[2];
        uint16_t *orow[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t16 = tlo + 32 * w + 16 * tt;  // the chunk's first token
            const int t = t16 + col;                 // this lane's token (B column, D column)
            live[tt] = t < te;
            const int tc = live[tt] ? t : tb;
            // the chunk's y tile (a chunk past the segment's end re-reads its first one)
            const int ch = chunk_off[n] + ((t16 < te ? t16 : tb) - tok_off[n]) / kC;
            const uint16_t *ytile = ybuf + ((int64_t)ch * H + h) * (kC * kD) + 8 * lane;
            orow[tt] = out + (int64_t)tc * rowst + (int64_t)h * kD;
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) yb[tt][ks] = *reinterpret_cast<const bf16x8 *>(ytile + 64 * 8 * ks);
#pragma unroll
            for (int p = 0; p < kD / 32; ++p) ov[tt][p] = *reinterpret_cast<const u32x4 *>(orow[tt] + 32 * p + 8 * g);
        }
        // two halves of the value channels, 64 each: 32 accumulator registers per lane
        // rather than 64 keep the kernel under 128 VGPRs, so two workgroups share a CU
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x4 acc[2][4];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[tt][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {  // each S_in fragment pair serves both token tiles
                    const int j = 4 * half + jj;
                    const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(&Shi[16 * j + col][32 * ks + 8 * g]);
                    const bf16x8 al = *reinterpret_cast<const bf16x8 *>(&Slo[16 * j + col][32 * ks + 8 * g]);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        acc[tt][jj] = mma32(ah, yb[tt][ks], acc[tt][jj]);
                        acc[tt][jj] = mma32(al, yb[tt][ks], acc[tt][jj]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // keep one k-step's LDS fragments live at a time
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if (live[tt]) {
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int p = 2 * half + pp;
                        const u32x4 o = ov[tt][p];
                        const f32x4 a0 = acc[tt][2 * pp], a1 = acc[tt][2 * pp + 1];
                        const f32x2 c0 = {bf_lo(o[0]) + a0[0], bf_hi(o[0]) + a0[1]};
                        const f32x2 c1 = {bf_lo(o[1]) + a0[2], bf_hi(o[1]) + a0[3]};
                        const f32x2 c2 = {bf_lo(o[2]) + a1[0], bf_hi(o[2]) + a1[1]};
                        const f32x2 c3 = {bf_lo(o[3]) + a1[2], bf_hi(o[3]) + a1[3]};
                        *reinterpret_cast<u32x4 *>(orow[tt] + 32 * p + 8 * g) =
                            u32x4{pk_bf16(c0), pk_bf16(c1), pk_bf16(c2), pk_bf16(c3)};
                    }
                }
            }
        }
    }
}

// token blocks of a segment spread over enough workgroups to fill the GPU about twice
static int64_t corr_blocks(const Problem &p)
{
    const int64_t per_seg = (p.lay.seg_len * kC + kCorrTok - 1) / kCorrTok;
    const int64_t want = (2 * kSegTargetGroups + p.lay.seg_max * p.H - 1) / (p.lay.seg_max * p.H);
    return want < per_seg ? want : per_seg;
}

bool fits_seg_finish(const Problem &p)
{
    return grid_fits(p.N * p.H, kD / kScanRows, 64 * kScanWaves) &&
           grid_fits(p.lay.seg_max * p.H, corr_blocks(p), 64 * kCorrWaves);
}

template <typename TSt>
static hipError_t launch_seg_finish_t(const Problem &p, hipStream_t s)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    const int32_t *seg = reinterpret_cast<const int32_t *>(p.ws + p.lay.seg_off);
    const float *sfin = reinterpret_cast<const float *>(p.ws + p.lay.sfin);
    const float *phi = reinterpret_cast<const float *>(p.ws + p.lay.phi);
    float *sin = reinterpret_cast<float *>(p.ws + p.lay.sin);
    hipLaunchKernelGGL(kseg_scan<TSt>, dim3((unsigned)(p.N * p.H), kD / kScanRows), dim3(64 * kScanWaves), 0, s,
                       (const TSt *)p.s0, (TSt *)p.s1, seg, p.H, sfin, phi, sin);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int64_t blocks = corr_blocks(p);
    hipLaunchKernelGGL(kseg_correct, dim3((unsigned)(p.lay.seg_max * p.H), (unsigned)blocks), dim3(64 * kCorrWaves),
                       0, s, (uint16_t *)p.out, (const uint16_t *)(p.ws + p.lay.ybuf), (const float *)sin, tok, chk, seg,
                       (int)p.N, p.H, (int)p.lay.seg_len, (int)p.lay.seg_first);
    return hipGetLastError();
}

hipError_t launch_seg_finish(const Problem &p, hipStream_t s)
{
    return p.st_bf16 ? launch_seg_finish_t<uint16_t>(p, s) : launch_seg_finish_t<float>(p, s);
}

}  // namespace kda
