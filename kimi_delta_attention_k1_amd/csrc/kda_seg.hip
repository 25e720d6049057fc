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
// kseg_scan walks that chain over the segments of each (sequence, head) with
// split-bf16 matrix-core products; kseg_correct adds S_in y_t to the outputs of every
// segment after the first.
#include "kda_mfma_common.h"

namespace kda {

constexpr int kScanRows = 16;   // value rows (state rows) per scan workgroup
constexpr int kScanWaves = 8;   // wave w: key channels [16w, 16w + 16)
constexpr int kScanDepth = 2;   // segments whose Phi and S0 tiles are in flight ahead of the chain
constexpr int kScanLd = kD + 8; // padded LDS row (bf16)

// One workgroup (8 waves) per (sequence, head, 16 value rows v). Each step forms the
// transposed chain S^T <- Phi_g^T S^T + S0_g^T: wave w owns key channels [16w, 16w+16)
// as the rows of a 16x16 tile whose columns are the 16 value rows. Phi_g^T is the A
// operand, read straight from HBM as split-bf16 tiles the single pass stored in this
// operand order (kScanDepth segments ahead of the chain); S^T is the B operand, the
// previous step's tile in LDS as bf16 hi and lo halves, double-buffered so that one
// barrier per step suffices. Three products per 32-channel k step (hi hi, lo hi,
// hi lo) carry about 16 bits of each operand; the sums and S0 stay fp32. A lane ends
// each step with four consecutive key channels of one value row: S0 comes in and S_in
// goes out as one 1 KB block per wave, the final state as 16-byte pieces.
template <typename TSt>
__global__ __launch_bounds__(64 * kScanWaves) void kseg_scan(const TSt *s0, TSt *s1,
                                                             const int32_t *__restrict__ seg_off, int H,
                                                             const float *__restrict__ sfin,
                                                             const uint16_t *__restrict__ phi, float *__restrict__ sin)
{
    __shared__ __attribute__((aligned(16))) uint16_t Sh[2][kScanRows][kScanLd];  // [buffer][v][key] hi
    __shared__ __attribute__((aligned(16))) uint16_t Sl[2][kScanRows][kScanLd];  // lo
    const int n = blockIdx.x / H, h = blockIdx.x % H, r0 = blockIdx.y * kScanRows;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
    const int first = seg_off[n], G = seg_off[n + 1] - first;
    const int64_t mat = (int64_t)kD * kD;
    // this lane's four state elements, value row r0 + col, key channels 16w + 4g .. +3:
    // their offset in a row-major state (initial and final) and in the tile order of
    // the workspace's S0 and S_in (one 1 KB block per wave)
    const int64_t eoff = (int64_t)(r0 + col) * kD + 16 * w + 4 * g;
    const int64_t toff = state_tile(r0 + col, 16 * w + 4 * g);
    auto sg_base = [&](int gi) { return ((int64_t)(first + gi) * H + h) * mat; };
    // segment gi's Phi^T tiles of this wave: k step ks, hi then lo, 1 KB per wave
    auto load_step = [&](int gi, bf16x8 (&ph)[4], bf16x8 (&pl)[4], f32x4 &z) {
        const uint16_t *P = phi + 2 * sg_base(gi) + (int64_t)w * (4 * 2 * 512) + lane * 8;  // hi and lo: 2 per element
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            ph[ks] = *reinterpret_cast<const bf16x8 *>(P + (2 * ks) * 512);
            pl[ks] = *reinterpret_cast<const bf16x8 *>(P + (2 * ks + 1) * 512);
        }
        z = *reinterpret_cast<const f32x4 *>(sfin + sg_base(gi) + toff);
    };
    // the state entering segment 1: segment 0's run started from the initial state
    f32x4 S;
    if (G > 0)
        S = *reinterpret_cast<const f32x4 *>(sfin + sg_base(0) + toff);
    else
        S = s0 ? ld_state4(s0 + ((int64_t)n * H + h) * mat + eoff) : f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ph[kScanDepth][4], pl[kScanDepth][4];
    f32x4 z[kScanDepth];
    // loads past the last segment re-read it (clamped): every step issues the same loads
    if (G > 1) {
#pragma unroll
        for (int d = 0; d < kScanDepth; ++d) load_step(min(1 + d, G - 1), ph[d], pl[d], z[d]);
    }
    // S as the next step's B operand: value row col, key channels 16w + 4g .. +3
    auto put = [&](int buf, f32x4 x) {
        bf16x4 hi, lo;
        split4t_packed(x, hi, lo);
        *reinterpret_cast<bf16x4 *>(&Sh[buf][col][16 * w + 4 * g]) = hi;
        *reinterpret_cast<bf16x4 *>(&Sl[buf][col][16 * w + 4 * g]) = lo;
    };
    if (G > 1) {
        *reinterpret_cast<f32x4 *>(sin + sg_base(1) + toff) = S;
        put(0, S);
    }
    __syncthreads();
    auto step = [&](int gi, bf16x8 (&pa)[4], bf16x8 (&pb)[4], f32x4 &zz) {
        const int buf = (gi - 1) & 1;
        f32x4 a0 = zz, a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&Sh[buf][col][32 * ks + 8 * g]);
            const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&Sl[buf][col][32 * ks + 8 * g]);
            a0 = mma32(pa[ks], bh, a0);
            a1 = mma32(pb[ks], bh, a1);
            a2 = mma32(pa[ks], bl, a2);
        }
        load_step(min(gi + kScanDepth, G - 1), pa, pb, zz);  // the buffers are free once used
        S = a0 + (a1 + a2);
        if (gi + 1 < G) {
            *reinterpret_cast<f32x4 *>(sin + sg_base(gi + 1) + toff) = S;
            put(buf ^ 1, S);
        }
        __syncthreads();  // the next step reads the other buffer; this one is rewritten after it
    };
    // unrolled over the buffers, so each step addresses its own statically
    int gi = 1;
#pragma unroll 1
    for (; gi + kScanDepth - 1 < G; gi += kScanDepth) {
#pragma unroll
        for (int d = 0; d < kScanDepth; ++d) step(gi + d, ph[d], pl[d], z[d]);
    }
#pragma unroll
    for (int d = 0; d + 1 < kScanDepth; ++d)
        if (gi + d < G) step(gi + d, ph[d], pl[d], z[d]);
    if (s1) st_state4(s1 + ((int64_t)n * H + h) * mat + eoff, S);
}

constexpr int kCorrWaves = 8;
constexpr int kCorrTok = 32 * kCorrWaves;  // tokens per workgroup

// LDS row of value channel r = 32p + 8g + 4u + i: row 16 (2p + u) + 4g + i. Result tiles
// 2p and 2p + 1 then hold channels 32p + 8g + (0..3) and (4..7) in lane group g, so a
// lane reads and writes eight consecutive output channels (16 bytes) at once.
__device__ __forceinline__ int corr_row(int r) { return (r & ~31) + 16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3); }
// LDS column of key channel c = 32 ks + 16 u + 4 g + i: column 32 ks + 8 g + 4 u + i, the
// order in which the single pass stores a y tile (lane group g of k step ks holds
// channels 32 ks + 4 g + (0..3), then 32 ks + 16 + 4 g + (0..3))
__device__ __forceinline__ int corr_col(int c) { return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3); }
// LDS element of (row, column) in the unpadded bf16 S_in halves: the 16-byte pieces of a
// row are XOR-swizzled by its low three bits, so eight lanes reading the same piece of
// eight rows (an A-operand read) hit eight different 16-byte bank groups
__device__ __forceinline__ int corr_lds(int row, int col) { return row * kD + ((((col >> 3) ^ row) & 7) | ((col >> 3) & ~7)) * 8 + (col & 7); }
// 16-byte piece `piece` (0..7) of token row `tr` (0..15) of a wave's output staging buffer
// (half of each token's output row), swizzled the same way
__device__ __forceinline__ int corr_stage(int tr, int piece) { return tr * 8 + ((piece ^ tr) & 7); }

// o_t += S_in y_t for every segment after the first. Workgroup (segment, head, j)
// splits S_in once into bf16 hi and lo halves in LDS, then walks the segment's
// token blocks j, j + gridDim.y, ... of 256 tokens: wave w takes 32 tokens (two
// chunks) and forms (S_in y^T) for them as 16x16 tiles (rows: value channels in the
// order corr_row gives, columns: tokens), so each lane ends with eight consecutive
// value channels of one token. The y of a chunk is one 4 KB tile in operand order.
// at least four waves per SIMD (at most 128 VGPRs): two 8-wave workgroups per CU
__global__ __launch_bounds__(64 * kCorrWaves, 4) void kseg_correct(uint16_t *__restrict__ out,
                                                                 const uint16_t *__restrict__ ybuf,
                                                                 const float *__restrict__ sin,
                                                                 const int32_t *__restrict__ tok_off,
                                                                 const int32_t *__restrict__ chunk_off,
                                                                 const int32_t *__restrict__ seg_off, int N, int H,
                                                                 int seg_len, int seg_first)
{
    // 2 x 32 KB of S_in halves and 2 KB of output staging per wave: 80 KB, two workgroups per CU
    __shared__ __attribute__((aligned(16))) uint16_t Shi[kD * kD];
    __shared__ __attribute__((aligned(16))) uint16_t Slo[kD * kD];
    __shared__ __attribute__((aligned(16))) u32x4 Ost[kCorrWaves][16 * 8];
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
        // element 4i of the tile order: value row 16 y + L % 16, key channels 16 w + 4 (L / 16)
        // .. +3 for i = (8 y + w) 64 + L
        const int L = i & 63, yw = i >> 6;
        const int r = 16 * (yw >> 3) + (L & 15), c = 16 * (yw & 7) + 4 * (L >> 4);
        const u32x4 u = __builtin_bit_cast(u32x4, x);
        // hi truncated (x - hi is exact in fp32), lo the remainder rounded
        const u32x2 hi = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u), __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
        const f32x2 r01 = {x[0] - __uint_as_float(u[0] & 0xffff0000u), x[1] - __uint_as_float(u[1] & 0xffff0000u)};
        const f32x2 r23 = {x[2] - __uint_as_float(u[2] & 0xffff0000u), x[3] - __uint_as_float(u[3] & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(&Shi[corr_lds(corr_row(r), corr_col(c))]) = hi;
        *reinterpret_cast<u32x2 *>(&Slo[corr_lds(corr_row(r), corr_col(c))]) = u32x2{pk_bf16(r01), pk_bf16(r23)};
    }
    __syncthreads();

    const int64_t rowst = (int64_t)H * kD;
#pragma unroll 1
    for (int tlo = tb + blockIdx.y * kCorrTok; tlo < te; tlo += gridDim.y * kCorrTok) {
        // every load of the block's two token tiles is issued before any product, so
        // each wave keeps 2 x (512 B y + 256 B o) per lane-row in flight at once
        bf16x8 yb[2][kD / 32];
        // the outputs as whole half rows: ov[tt][k] holds, for lane L, 16 bytes at byte
        // 128 half + 16 (L % 8) of token t16 + 8k + L / 8 (rows past the end: the
        // segment's first, never stored); the second half is loaded while the first
        // half's products run
        u32x4 ov[2][2];
        uint16_t *orow[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t16 = tlo + 32 * w + 16 * tt;  // the chunk's first token
            // the chunk's y tile (a chunk past the segment's end re-reads its first one)
            const int ch = chunk_off[n] + ((t16 < te ? t16 : tb) - tok_off[n]) / kC;
            const uint16_t *ytile = ybuf + ((int64_t)ch * H + h) * (kC * kD) + 8 * lane;
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) yb[tt][ks] = *reinterpret_cast<const bf16x8 *>(ytile + 64 * 8 * ks);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int t = t16 + 8 * k + (lane >> 3);
                orow[tt][k] = out + (int64_t)(t < te ? t : tb) * rowst + (int64_t)h * kD + 8 * (lane & 7);
                ov[tt][k] = *reinterpret_cast<const u32x4 *>(orow[tt][k]);
            }
        }
        u32x4 *const stage = Ost[w];
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
                    const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(&Shi[corr_lds(16 * j + col, 32 * ks + 8 * g)]);
                    const bf16x8 al = *reinterpret_cast<const bf16x8 *>(&Slo[corr_lds(16 * j + col, 32 * ks + 8 * g)]);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        acc[tt][jj] = mma32(ah, yb[tt][ks], acc[tt][jj]);
                        acc[tt][jj] = mma32(al, yb[tt][ks], acc[tt][jj]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // keep one k-step's LDS fragments live at a time
            }
            u32x4 on[2][2];  // the second half's rows, in flight during this half's epilogue
            if (half == 0) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int k = 0; k < 2; ++k) on[tt][k] = *reinterpret_cast<const u32x4 *>(orow[tt][k] + 64);
            }
            // this half of each token's outputs, through the wave's staging buffer: in as
            // whole half rows, out to the products' lanes (token col, channels 32p + 8g .. +7,
            // bytes 64 pp + 16 g of the half row), back, and stored as whole half rows. A
            // wave's LDS operations complete in order, so no wait is needed in between.
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int k = 0; k < 2; ++k) stage[corr_stage(8 * k + (lane >> 3), lane & 7)] = ov[tt][k];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const u32x4 o = stage[corr_stage(col, 4 * pp + g)];
                    const f32x4 a0 = acc[tt][2 * pp], a1 = acc[tt][2 * pp + 1];
                    const f32x2 c0 = {bf_lo(o[0]) + a0[0], bf_hi(o[0]) + a0[1]};
                    const f32x2 c1 = {bf_lo(o[1]) + a0[2], bf_hi(o[1]) + a0[3]};
                    const f32x2 c2 = {bf_lo(o[2]) + a1[0], bf_hi(o[2]) + a1[1]};
                    const f32x2 c3 = {bf_lo(o[3]) + a1[2], bf_hi(o[3]) + a1[3]};
                    stage[corr_stage(col, 4 * pp + g)] = u32x4{pk_bf16(c0), pk_bf16(c1), pk_bf16(c2), pk_bf16(c3)};
                }
                const int t16 = tlo + 32 * w + 16 * tt;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const u32x4 o = stage[corr_stage(8 * k + (lane >> 3), lane & 7)];
                    if (t16 + 8 * k + (lane >> 3) < te) *reinterpret_cast<u32x4 *>(orow[tt][k] + 64 * half) = o;
                }
            }
            if (half == 0) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int k = 0; k < 2; ++k) ov[tt][k] = on[tt][k];
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
    const uint16_t *phi = reinterpret_cast<const uint16_t *>(p.ws + p.lay.phi);
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
