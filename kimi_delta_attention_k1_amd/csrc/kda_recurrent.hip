// kda_recurrent.hip -- token-by-token KDA forward for decode and short sequences.
//
// Evaluates the boxed KDA recurrence of the Doubleword page "You Could Have Come Up
// with Kimi Delta Attention" (section 4) directly, one token at a time, in fp32:
//   S~ = S Diag(alpha_t);  e = beta_t (v_t - S~ k_t);  S = S~ + e k_t^T;  o_t = S (s q_t)
// with alpha_t = exp(lb sigmoid(g_raw_t)), beta_t = sigmoid(beta_raw_t) and q, k
// L2-normalised, as in the other paths. Value rows of S evolve independently given
// the token's q, k, alpha, beta (the update is row-wise), so the state splits into
// 16-row slices that need no communication (Doubleword section 6.3 makes the same
// observation for the chunked solve).
//
// Grid: one 128-thread workgroup per (sequence, head, 16-row value slice). Lane l of
// wave w owns rows 8w + 2i + l/32 (i = 0..3) of the slice at key channels
// [4 (l%32), 4 (l%32) + 4): 16 fp32 state values in registers. A wave's eight rows are
// 4 KB in one piece, and each of its four state loads and stores moves 1 KB of it in
// one piece (lane l at byte 16 l, then 1 KB further), whole cache lines: with a lane's
// 16 channels of one row as 64 contiguous bytes, each access touched 16-byte pieces of
// 32 lines, and decode streamed the state 18% slower.
// Tokens go in blocks of 8: the block's activations (q^ s, k^, alpha, beta and the
// slice's v) are computed by all 128 threads at once into LDS, then the serial loop
// applies the recurrence token by token with 32-lane reductions for S k and S q.
// With T = 1 (decode) the kernel is one pass over the state: 128 KiB of HBM traffic
// per (sequence, head) for an fp32 state.
#include "kda_mfma_common.h"

namespace kda {

constexpr int kRThreads = 128;
constexpr int kRRows = 16;  // value rows per workgroup
constexpr int kRBlock = 8;  // tokens per activation block

template <typename T> struct InVec;
template <> struct InVec<uint16_t> {
    // 16 consecutive elements as fp32
    static __device__ __forceinline__ void load16(const uint16_t *p, float *x)
    {
        const uint4 a = reinterpret_cast<const uint4 *>(p)[0], b = reinterpret_cast<const uint4 *>(p)[1];
        const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <> struct InVec<float> {
    static __device__ __forceinline__ void load16(const float *p, float *x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = reinterpret_cast<const float4 *>(p)[i];
            x[4 * i] = a.x;
            x[4 * i + 1] = a.y;
            x[4 * i + 2] = a.z;
            x[4 * i + 3] = a.w;
        }
    }
};

// sum over the 8 lanes l with equal l / 8 (lanes differ in bits 0-2)
__device__ __forceinline__ float sum8(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x;
}
// sum over the 32 lanes l with equal l / 32
__device__ __forceinline__ float sum32(float x)
{
    x = sum8(x);
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    return x;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// sigmoid and exp from 2^x and a reciprocal (v_exp_f32, v_rcp_f32). The gate's
// exponent lb sigmoid(g) log2(e) has magnitude below 15, so its rounding moves alpha
// by less than 1e-6 relative, and slow decays, where errors could pile up over many
// tokens, have small exponents.
__device__ __forceinline__ float sigmoid2(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <typename TIn, typename TSt>
__global__ __launch_bounds__(kRThreads) void kr_recurrent(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                          const TIn *__restrict__ v, const TIn *__restrict__ graw,
                                                          const TIn *__restrict__ braw, const TSt *s0, TSt *s1,
                                                          TIn *__restrict__ out, const int32_t *__restrict__ tok_off,
                                                          int H, float lb, float scale, int scalar_gate)
{
    __shared__ __attribute__((aligned(16))) float sQ[kRBlock][kD], sK[kRBlock][kD], sA[kRBlock][kD];
    __shared__ float sB[kRBlock], sV[kRBlock][kRRows];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = blockIdx.x % (kD / kRRows);
    const int pair = blockIdx.x / (kD / kRRows);
    const int n = pair / H, h = pair % H;
    const int tb = tok_off[n], te = tok_off[n + 1];

    // state: rows 8w + 2i + hr of this slice (s[i]), key channels [4 c4, 4 c4 + 4);
    // row 8w + hr at channel 4 c4 is element 4 l of the wave's 4 KB, row 8w + 2i + hr
    // 256 i elements further
    const int hr = lane >> 5, c4 = lane & 31;
    const int64_t soff = (((int64_t)n * H + h) * kD + kRRows * slice + 8 * w) * kD + 4 * lane;
    f32x4 s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = s0 != nullptr ? ld_state4(s0 + soff + 2 * kD * i) : f32x4{0.f, 0.f, 0.f, 0.f};

    // activation work split: thread (at, ap) handles token at of the block, channels [16 ap, 16 ap + 16)
    const int at = tid >> 3, ap = tid & 7;
    const float lb2 = lb * kLog2e;
#pragma unroll 1
    for (int t0 = tb; t0 < te; t0 += kRBlock) {
        const int nb = min(kRBlock, te - t0);
        if (at < nb) {
            const int64_t row = ((int64_t)(t0 + at) * H + h) * kD + 16 * ap;
            float qx[16], kx[16];
            InVec<TIn>::load16(q + row, qx);
            InVec<TIn>::load16(k + row, kx);
            float nq = 0.f, nk = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                nq += qx[i] * qx[i];
                nk += kx[i] * kx[i];
            }
            nq = sum8(nq);
            nk = sum8(nk);
            const float rq = scale / sqrtf(nq + kL2Eps), rk = 1.0f / sqrtf(nk + kL2Eps);
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                *reinterpret_cast<float4 *>(&sQ[at][16 * ap + i]) =
                    make_float4(qx[i] * rq, qx[i + 1] * rq, qx[i + 2] * rq, qx[i + 3] * rq);
                *reinterpret_cast<float4 *>(&sK[at][16 * ap + i]) =
                    make_float4(kx[i] * rk, kx[i + 1] * rk, kx[i + 2] * rk, kx[i + 3] * rk);
            }
            if (ap == 0) sB[at] = sigmoid2(ld_elem(braw, (int64_t)(t0 + at) * H + h));
            if (ap < 2) {  // the slice's 16 v values of token at
                const int64_t vo = ((int64_t)(t0 + at) * H + h) * kD + kRRows * slice + 8 * ap;
#pragma unroll
                for (int i = 0; i < 8; ++i) sV[at][8 * ap + i] = ld_elem(v, vo + i);
            }
        }
        // the gates, one (token, channel) per thread and pass: a single decode token
        // still spreads over all 128 threads
        for (int e = tid; e < nb * kD; e += kRThreads) {
            const int j = e / kD, c = e % kD;
            // a scalar gate ([T][H]) serves every channel
            const int64_t th = (int64_t)(t0 + j) * H + h;
            const float g = ld_elem(graw, scalar_gate ? th : th * kD + c);
            sA[j][c] = __builtin_amdgcn_exp2f(lb2 * sigmoid2(g));
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < nb; ++j) {
            const f32x4 av = *reinterpret_cast<const f32x4 *>(&sA[j][4 * c4]);
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(&sK[j][4 * c4]);
            const f32x4 qv = *reinterpret_cast<const f32x4 *>(&sQ[j][4 * c4]);
            float p[4], o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // forget, then predict: (S Diag(alpha) k)[row]
                s[i] *= av;
                p[i] = dot4(s[i], kv);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = sum32(p[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = sB[j] * (sV[j][8 * w + 2 * i + hr] - p[i]);  // correct
                s[i] += e * kv;                                               // write, then read
                o[i] = dot4(s[i], qv);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sum32(o[i]);
            if (c4 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st_elem(out, ((int64_t)(t0 + j) * H + h) * kD + kRRows * slice + 8 * w + 2 * i + hr, o[i]);
            }
        }
        __syncthreads();  // the next block overwrites the activations
    }
    if (s1 != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st_state4(s1 + soff + 2 * kD * i, s[i]);
    }
}

template <typename TIn, typename TSt>
static hipError_t launch_recurrent_t(const Problem &p, hipStream_t st)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const unsigned grid = (unsigned)(p.N * p.H * (kD / kRRows));
    hipLaunchKernelGGL((kr_recurrent<TIn, TSt>), dim3(grid), dim3(kRThreads), 0, st, (const TIn *)p.q,
                       (const TIn *)p.k, (const TIn *)p.v, (const TIn *)p.g, (const TIn *)p.beta, (const TSt *)p.s0,
                       (TSt *)p.s1, (TIn *)p.out, tok, p.H, p.lb, p.scale, (int)p.scalar_gate);
    return hipGetLastError();
}

bool fits_recurrent(const Problem &p) { return grid_fits(p.N * p.H * (kD / kRRows), 1, kRThreads); }

hipError_t launch_recurrent(const Problem &p, hipStream_t st)
{
    if (p.io_bf16)
        return p.st_bf16 ? launch_recurrent_t<uint16_t, uint16_t>(p, st) : launch_recurrent_t<uint16_t, float>(p, st);
    return p.st_bf16 ? launch_recurrent_t<float, uint16_t>(p, st) : launch_recurrent_t<float, float>(p, st);
}

}  // namespace kda
