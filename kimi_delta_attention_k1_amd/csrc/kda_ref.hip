// kda_ref.hip -- chunk map kernel and the fp32 reference path of the KDA forward.
//
// The fp32 path is the plain, slow GPU rendering of the chunkwise method on the
// Doubleword page "You Could Have Come Up with Kimi Delta Attention",
// section 6: per chunk the prefix-summed log-decays (6.6), the causal
// coefficients rho and chi (6.3, 6.5), the unit-lower-triangular inverse A^kk
// (6.3), and the chunk state scan (6.4) with outputs (6.5). It runs for fp32
// I/O and for bf16 I/O when the caller asks for fp32 compute. Every product is
// an fp32 FMA loop, and decay ratios are exp of log-decay differences.
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------------------
// K0: sanitised token offsets and chunk offsets, one workgroup.
// With cu_seqlens: tok_off[n] = min(T_tot, max_{m<=n} clamp(cu[m], 0, T_tot)),
// tok_off[0] = 0, tok_off[N] = T_tot; flag = 1 iff cu already had that form.
// Without: tok_off[n] = n*T. chunk_off is the exclusive scan of
// ceil((tok_off[n+1]-tok_off[n]) / 16); on the segmented path seg_off is the
// exclusive scan of the segments of each sequence (seg_count); on the single pass,
// order lists the sequences longest first.
// ---------------------------------------------------------------------------
constexpr int kMapThreads = 1024;

constexpr int kMapWaves = kMapThreads / 64;

// inclusive scan (sum, or running max) over the workgroup: lane shuffles within each
// wave, then one wave scans the wave totals; sh[kMapThreads] receives the total
__device__ __forceinline__ int block_scan_incl(int x, int *sh, bool is_max)
{
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int ident = is_max ? INT32_MIN : 0;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x = is_max ? max(x, y) : x + y;
    }
    if (lane == 63) sh[w] = x;  // wave totals
    __syncthreads();
    if (w == 0) {
        int v = lane < kMapWaves ? sh[lane] : ident;
        for (int off = 1; off < kMapWaves; off <<= 1) {
            const int y = __shfl_up(v, off, 64);
            if (lane >= off) v = is_max ? max(v, y) : v + y;
        }
        if (lane < kMapWaves) sh[kMapWaves + lane] = v;  // inclusive over waves
        if (lane == kMapWaves - 1) sh[kMapThreads] = v;  // broadcast slot
    }
    __syncthreads();
    if (w > 0) {
        const int y = sh[kMapWaves + w - 1];
        x = is_max ? max(x, y) : x + y;
    }
    __syncthreads();  // the caller reads sh[kMapThreads]; the next scan rewrites sh
    return x;
}

__global__ __launch_bounds__(kMapThreads) void k0_chunk_map(const int32_t *__restrict__ cu, int N, int T,
                                                             int T_tot, int32_t *__restrict__ hdr,
                                                             int32_t *__restrict__ tok_off,
                                                             int32_t *__restrict__ chunk_off, int seg_len,
                                                             int seg_first, int32_t *__restrict__ seg_off,
                                                             int32_t *__restrict__ order)
{
    __shared__ int sh[kMapThreads + 1];
    // with N <= kMapThreads every offset is also kept here, so later passes read LDS
    // rather than global memory just written by other threads
    __shared__ int ltok[kMapThreads + 1], lchk[kMapThreads + 1];
    const bool small = N <= kMapThreads;
    const int t = threadIdx.x;
    __shared__ int bad;
    if (t == 0) bad = 0;
    __syncthreads();
    // pass 1: token offsets (prefix max of clamped entries)
    int carry = 0;
    for (int base = 0; base <= N; base += kMapThreads) {
        const int n = base + t;
        int x = carry;
        if (n <= N) {
            if (cu) {
                int raw = cu[n];
                int c = min(max(raw, 0), T_tot);
                if (n == N) c = T_tot;
                if (n == 0) c = 0;
                bool ok = (raw == c) && (n == 0 || raw >= cu[n - 1]);
                if (!ok) atomicOr(&bad, 1);
                x = max(c, carry);
            } else {
                x = n * T;
            }
        }
        int s = block_scan_incl(x, sh, true);
        if (n <= N) tok_off[n] = s;
        if (small && n <= N) ltok[n] = s;
        carry = sh[kMapThreads];
        __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    // pass 2: chunk offsets
    carry = 0;
    for (int base = 0; base <= N; base += kMapThreads) {
        const int n = base + t;
        int cnt = 0;
        if (n < N) cnt = small ? (ltok[n + 1] - ltok[n] + kC - 1) / kC : (tok_off[n + 1] - tok_off[n] + kC - 1) / kC;
        int s = block_scan_incl(cnt, sh, false);
        if (n <= N) chunk_off[n] = carry + s - cnt;  // exclusive
        if (small && n <= N) lchk[n] = carry + s - cnt;
        carry += sh[kMapThreads];
        __syncthreads();
    }
    if (seg_off != nullptr) {
        // pass 3: segment offsets, the exclusive scan of the segments per sequence
        __threadfence_block();
        __syncthreads();
        carry = 0;
        for (int base = 0; base <= N; base += kMapThreads) {
            const int n = base + t;
            int cnt = 0;
            if (n < N) cnt = seg_count(small ? lchk[n + 1] - lchk[n] : chunk_off[n + 1] - chunk_off[n], seg_len, seg_first);
            int s = block_scan_incl(cnt, sh, false);
            if (n <= N) seg_off[n] = carry + s - cnt;
            carry += sh[kMapThreads];
            __syncthreads();
        }
    }
    if (order != nullptr) {
        // pass 4: sequences by chunk count, longest first (ties: lower index first);
        // beyond one sequence per thread the input order is kept
        __threadfence_block();
        __syncthreads();
        if (N <= kMapThreads) {
            if (t < N) {
                const int ct = lchk[t + 1] - lchk[t];
                int rank = 0;
                for (int m = 0; m < N; ++m) {
                    const int cm = lchk[m + 1] - lchk[m];
                    rank += (cm > ct || (cm == ct && m < t)) ? 1 : 0;
                }
                order[rank] = t;
            }
        } else {
            for (int n = t; n < N; n += kMapThreads) order[n] = n;
        }
    }
    if (t == 0) hdr[0] = bad ? 0 : 1;
}

// inclusive scan (sum, or running max) over one wave
__device__ __forceinline__ int wave_scan_incl(int x, bool is_max)
{
    const int lane = threadIdx.x & 63;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x = is_max ? max(x, y) : x + y;
    }
    return x;
}

// K0 as one wave and no barrier: lane l holds entries E l .. E l + E - 1 of every
// offset array (N + 1 <= 64 E), scanned within the lane and then across the wave;
// the longest-first order comes from one comparison loop over the N sequences per
// entry. The same results as k0_chunk_map in about half the time: a small call
// spends about as long in K0 as in its scan kernel.
template <int E>
__global__ __launch_bounds__(64) void k0_chunk_map_wave(const int32_t *__restrict__ cu, int N, int T, int T_tot,
                                                      int32_t *__restrict__ hdr, int32_t *__restrict__ tok_off,
                                                      int32_t *__restrict__ chunk_off, int seg_len, int seg_first,
                                                      int32_t *__restrict__ seg_off, int32_t *__restrict__ order)
{
    const int lane = threadIdx.x, n0 = E * lane;
    int tok[E], cnt[E];
    bool bad = false;
    // token offsets: the running maximum of the clamped entries
    int run = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int n = n0 + e;
        int x = 0;
        if (n <= N) {
            if (cu) {
                const int raw = cu[n];
                int c = min(max(raw, 0), T_tot);
                if (n == N) c = T_tot;
                if (n == 0) c = 0;
                bad |= !((raw == c) && (n == 0 || raw >= cu[n - 1]));
                x = c;
            } else {
                x = n * T;
            }
        }
        run = max(run, x);
        tok[e] = run;
    }
    const int before = __shfl_up(wave_scan_incl(run, true), 1, 64);  // max over the lanes below
#pragma unroll
    for (int e = 0; e < E; ++e) tok[e] = lane > 0 ? max(tok[e], before) : tok[e];
    // chunks per sequence: the next entry is this lane's next one or the next lane's first
    const int next_first = __shfl_down(tok[0], 1, 64);
    int csum = 0, ssum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int n = n0 + e;
        const int nxt = e + 1 < E ? tok[e + 1] : next_first;
        cnt[e] = n < N ? (nxt - tok[e] + kC - 1) / kC : 0;
        csum += cnt[e];
        ssum += (n < N && seg_off != nullptr) ? seg_count(cnt[e], seg_len, seg_first) : 0;
    }
    int cex = wave_scan_incl(csum, false) - csum, sex = wave_scan_incl(ssum, false) - ssum;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int n = n0 + e;
        if (n <= N) {
            tok_off[n] = tok[e];
            chunk_off[n] = cex;
            if (seg_off != nullptr) seg_off[n] = sex;
        }
        if (seg_off != nullptr && n < N) sex += seg_count(cnt[e], seg_len, seg_first);
        cex += cnt[e];
    }
    if (order != nullptr) {
        // sequences by chunk count, longest first (ties: lower index first): each
        // entry counts the sequences ranked before it
        int rank[E] = {};
        for (int j = 0; j * E < N; ++j) {
#pragma unroll
            for (int f = 0; f < E; ++f) {
                const int m = E * j + f, cm = __shfl(cnt[f], j, 64);
                if (m < N) {
#pragma unroll
                    for (int e = 0; e < E; ++e) rank[e] += (cm > cnt[e] || (cm == cnt[e] && m < n0 + e)) ? 1 : 0;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (n0 + e < N) order[rank[e]] = n0 + e;
    }
    const bool any_bad = __ballot(bad) != 0;
    if (lane == 0) hdr[0] = any_bad ? 0 : 1;
}

hipError_t launch_chunk_map(const Problem &p, hipStream_t s)
{
    int32_t *hdr = reinterpret_cast<int32_t *>(p.ws);
    int32_t *tok = reinterpret_cast<int32_t *>(p.ws + p.lay.tok_off);
    int32_t *chk = reinterpret_cast<int32_t *>(p.ws + p.lay.chunk_off);
    int32_t *seg = p.lay.seg_len > 0 ? reinterpret_cast<int32_t *>(p.ws + p.lay.seg_off) : nullptr;
    int32_t *ord = p.lay.order > 0 ? reinterpret_cast<int32_t *>(p.ws + p.lay.order) : nullptr;
    // one wave up to 127 sequences (two entries per lane): measured faster than the
    // workgroup kernel there, slower from 256 sequences on (16 entries per lane)
    const int ln = (int)p.lay.seg_len, lf = (int)p.lay.seg_first, N = (int)p.N, T = (int)p.T, Tt = (int)p.T_tot;
    if (N < 64)
        hipLaunchKernelGGL(k0_chunk_map_wave<1>, dim3(1), dim3(64), 0, s, p.cu, N, T, Tt, hdr, tok, chk, ln, lf, seg,
                           ord);
    else if (N < 128)
        hipLaunchKernelGGL(k0_chunk_map_wave<2>, dim3(1), dim3(64), 0, s, p.cu, N, T, Tt, hdr, tok, chk, ln, lf, seg,
                           ord);
    else
        hipLaunchKernelGGL(k0_chunk_map, dim3(1), dim3(kMapThreads), 0, s, p.cu, N, T, Tt, hdr, tok, chk, ln, lf, seg,
                           ord);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 reference K1: one workgroup (256 threads) per (chunk, head).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_ref(float x) { return 1.0f / (1.0f + expf(-x)); }

template <typename TIn>
__global__ __launch_bounds__(256) void k1_ref(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                               const TIn *__restrict__ g, const TIn *__restrict__ beta,
                                               const int32_t *__restrict__ tok_off,
                                               const int32_t *__restrict__ chunk_off, int N, int H,
                                               int64_t n_c_max, float lb, float scale, int scalar_gate,
                                               char *__restrict__ units)
{
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    if (c >= chunk_off[N]) return;
    const int n = find_seq(chunk_off, N, c);
    const int t0 = tok_off[n] + (c - chunk_off[n]) * kC;
    const int len = min(kC, tok_off[n + 1] - t0);

    __shared__ float sq[kC][kD], sk[kC][kD], sG[kC][kD];
    __shared__ float sbeta[kC], snq[kC], snk[kC], sR[kC][kC], sAqk[kC][kC], sAb[kC][kC];

    for (int idx = tid; idx < kC * kD; idx += 256) {
        const int i = idx >> 7, d = idx & 127;
        float qv = 0.f, kv = 0.f, gv = 0.f;
        if (i < len) {
            const int64_t off = ((int64_t)(t0 + i) * H + h) * kD + d;
            qv = ld_elem(q, off);
            kv = ld_elem(k, off);
            // log-decay g = lb * sigmoid(g_raw); a scalar gate ([T][H]) serves every channel
            const int64_t goff = scalar_gate ? (int64_t)(t0 + i) * H + h : off;
            gv = lb * sigmoid_ref(ld_elem(g, goff));
        }
        sq[i][d] = qv;
        sk[i][d] = kv;
        sG[i][d] = gv;
    }
    if (tid < kC) sbeta[tid] = (tid < len) ? sigmoid_ref(ld_elem(beta, (int64_t)(t0 + tid) * H + h)) : 0.f;
    __syncthreads();
    if (tid < kD) {  // in-chunk prefix sums of log-decay, per key channel
        float acc = 0.f;
        for (int i = 0; i < kC; ++i) {
            acc += sG[i][tid];
            sG[i][tid] = acc;
        }
    } else if (tid < kD + 2 * kC) {  // squared norms
        const int i = (tid - kD) & (kC - 1);
        const bool isk = tid >= kD + kC;
        float acc = 0.f;
        for (int d = 0; d < kD; ++d) {
            float x = isk ? sk[i][d] : sq[i][d];
            acc += x * x;
        }
        (isk ? snk : snq)[i] = 1.0f / sqrtf(acc + kL2Eps);
    }
    __syncthreads();
    for (int idx = tid; idx < kC * kD; idx += 256) {
        const int i = idx >> 7, d = idx & 127;
        sq[i][d] *= snq[i];
        sk[i][d] *= snk[i];
    }
    __syncthreads();
    {  // rho_ij (j < i) and chi_ij (j <= i)
        const int i = tid >> 4, j = tid & 15;
        float r = 0.f, a = 0.f;
        if (j <= i) {
            for (int d = 0; d < kD; ++d) {
                const float kj = sk[j][d] * expf(sG[i][d] - sG[j][d]);
                r += sk[i][d] * kj;
                a += sq[i][d] * kj;
            }
        }
        sR[i][j] = (j < i) ? sbeta[i] * r : 0.f;
        sAqk[i][j] = (j <= i) ? scale * a : 0.f;
    }
    __syncthreads();
    if (tid < kC) {  // (I + R)^-1 column tid by forward substitution, times beta_j
        const int j = tid;
        float x[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            float s = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s -= sR[i][m] * x[m];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < kC; ++i) sAb[i][j] = x[i] * sbeta[j];
    }
    __syncthreads();
    char *u = units + ((int64_t)h * n_c_max + c) * kUnitF32.bytes;
    float *KB = reinterpret_cast<float *>(u + kUnitF32.kb);
    float *QB = reinterpret_cast<float *>(u + kUnitF32.qb);
    float *KE = reinterpret_cast<float *>(u + kUnitF32.ke);
    float *AB = reinterpret_cast<float *>(u + kUnitF32.ab);
    float *AQ = reinterpret_cast<float *>(u + kUnitF32.aq);
    float *GM = reinterpret_cast<float *>(u + kUnitF32.gm);
    for (int idx = tid; idx < kC * kD; idx += 256) {
        const int i = idx >> 7, d = idx & 127;
        const float Gi = sG[i][d], Gl = sG[kC - 1][d];
        KB[idx] = sk[i][d] * expf(Gi);
        QB[idx] = scale * sq[i][d] * expf(Gi);
        KE[idx] = sk[i][d] * expf(Gl - Gi);
    }
    AB[tid] = (&sAb[0][0])[tid];
    AQ[tid] = (&sAqk[0][0])[tid];
    if (tid < kD) GM[tid] = expf(sG[kC - 1][tid]);
}

// ---------------------------------------------------------------------------
// fp32 reference K2: one workgroup (128 threads) per (sequence, head); thread v
// owns value row S[v][:] (the value channels evolve independently). The state
// lives in LDS as sS[k][v] so each thread walks its own column.
// ---------------------------------------------------------------------------
template <typename TIn, typename TSt>
__global__ __launch_bounds__(128) void k2_ref(const TIn *__restrict__ v, const TSt *s0, TSt *s1,
                                               TIn *__restrict__ out, const int32_t *__restrict__ tok_off,
                                               const int32_t *__restrict__ chunk_off, int H,
                                               int64_t n_c_max, const char *__restrict__ units)
{
    const int n = blockIdx.x, h = blockIdx.y, vv = threadIdx.x;
    __shared__ float sS[kD][kD];
    __shared__ float sKB[kC][kD], sQB[kC][kD], sKE[kC][kD], sAB[kC][kC], sAQ[kC][kC], sGM[kD];
    const int64_t sbase = ((int64_t)n * H + h) * kD * kD + (int64_t)vv * kD;
    for (int kk = 0; kk < kD; ++kk) sS[kk][vv] = s0 ? ld_elem(s0, sbase + kk) : 0.f;

    const int c0 = chunk_off[n], nch = chunk_off[n + 1] - c0;
    const int tb = tok_off[n], te = tok_off[n + 1];
    for (int j = 0; j < nch; ++j) {
        const char *u = units + ((int64_t)h * n_c_max + c0 + j) * kUnitF32.bytes;
        const float *KB = reinterpret_cast<const float *>(u + kUnitF32.kb);
        const float *QB = reinterpret_cast<const float *>(u + kUnitF32.qb);
        const float *KE = reinterpret_cast<const float *>(u + kUnitF32.ke);
        for (int idx = vv; idx < kC * kD; idx += 128) {
            (&sKB[0][0])[idx] = KB[idx];
            (&sQB[0][0])[idx] = QB[idx];
            (&sKE[0][0])[idx] = KE[idx];
        }
        (&sAB[0][0])[vv] = reinterpret_cast<const float *>(u + kUnitF32.ab)[vv];
        (&sAB[0][0])[vv + 128] = reinterpret_cast<const float *>(u + kUnitF32.ab)[vv + 128];
        (&sAQ[0][0])[vv] = reinterpret_cast<const float *>(u + kUnitF32.aq)[vv];
        (&sAQ[0][0])[vv + 128] = reinterpret_cast<const float *>(u + kUnitF32.aq)[vv + 128];
        sGM[vv] = reinterpret_cast<const float *>(u + kUnitF32.gm)[vv];
        __syncthreads();
        const int t0 = tb + j * kC, len = min(kC, te - t0);
        float Eb[kC], E[kC], o[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            Eb[i] = (i < len) ? ld_elem(v, ((int64_t)(t0 + i) * H + h) * kD + vv) : 0.f;
            o[i] = 0.f;
        }
        for (int kk = 0; kk < kD; ++kk) {  // Ebar = v_i - S_c D_{0:i} k_i ; o partial = s S_c D_{0:i} q_i
            const float sv = sS[kk][vv];
#pragma unroll
            for (int i = 0; i < kC; ++i) {
                Eb[i] -= sKB[i][kk] * sv;
                o[i] += sQB[i][kk] * sv;
            }
        }
#pragma unroll
        for (int i = 0; i < kC; ++i) {  // E = A^kk Diag(beta) Ebar
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < kC; ++m) acc += sAB[i][m] * Eb[m];
            E[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < kC; ++i) {  // o_i += sum_j chi_ij e_j
            float acc = o[i];
#pragma unroll
            for (int m = 0; m < kC; ++m) acc += sAQ[i][m] * E[m];
            if (i < len) st_elem(out, ((int64_t)(t0 + i) * H + h) * kD + vv, acc);
        }
        for (int kk = 0; kk < kD; ++kk) {  // S_{c+1} = S_c D_{0:last} + E K^end
            float acc = sGM[kk] * sS[kk][vv];
#pragma unroll
            for (int i = 0; i < kC; ++i) acc += E[i] * sKE[i][kk];
            sS[kk][vv] = acc;
        }
        __syncthreads();
    }
    if (s1) {
        for (int kk = 0; kk < kD; ++kk) st_elem(s1, sbase + kk, sS[kk][vv]);
    }
}

template <typename TIn>
static hipError_t launch_prep_ref_t(const Problem &p, hipStream_t s)
{
    if (p.n_c_max == 0) return hipSuccess;
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    hipLaunchKernelGGL((k1_ref<TIn>), dim3((unsigned)p.n_c_max, p.H), dim3(256), 0, s, (const TIn *)p.q,
                       (const TIn *)p.k, (const TIn *)p.g, (const TIn *)p.beta, tok, chk, (int)p.N, p.H,
                       p.n_c_max, p.lb, p.scale, (int)p.scalar_gate, p.ws + p.lay.units);
    return hipGetLastError();
}

template <typename TIn, typename TSt>
static hipError_t launch_recur_ref_t(const Problem &p, hipStream_t s)
{
    const int32_t *tok = reinterpret_cast<const int32_t *>(p.ws + p.lay.tok_off);
    const int32_t *chk = reinterpret_cast<const int32_t *>(p.ws + p.lay.chunk_off);
    hipLaunchKernelGGL((k2_ref<TIn, TSt>), dim3((unsigned)p.N, p.H), dim3(128), 0, s, (const TIn *)p.v,
                       (const TSt *)p.s0, (TSt *)p.s1, (TIn *)p.out, tok, chk, p.H, p.n_c_max,
                       (const char *)(p.ws + p.lay.units));
    return hipGetLastError();
}

bool fits_ref(const Problem &p) { return grid_fits(p.n_c_max, p.H, 256) && grid_fits(p.N, p.H, 128); }

hipError_t launch_prep_ref(const Problem &p, hipStream_t s)
{
    return p.io_bf16 ? launch_prep_ref_t<uint16_t>(p, s) : launch_prep_ref_t<float>(p, s);
}

hipError_t launch_recur_ref(const Problem &p, hipStream_t s)
{
    if (p.io_bf16)
        return p.st_bf16 ? launch_recur_ref_t<uint16_t, uint16_t>(p, s) : launch_recur_ref_t<uint16_t, float>(p, s);
    return p.st_bf16 ? launch_recur_ref_t<float, uint16_t>(p, s) : launch_recur_ref_t<float, float>(p, s);
}

}  // namespace kda
