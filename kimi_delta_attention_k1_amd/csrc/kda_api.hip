// kda_api.hip -- host side of the C ABI declared in include/kda.h: argument
// validation (pure host code, nothing touches the GPU before it passes),
// workspace carve-up and the kernel launches on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

using kda::Problem;
using kda::WsLayout;

constexpr int kVersion = 200;  // 0.2.0

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};
Range range_of(const void *p, size_t bytes)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, p ? a + bytes : a};
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

enum Path { kSplit, kFused, kRecurrent, kSeg };

struct Shape {
    int64_t T_tot, n_c_max;
    bool f32_path;
    Path path;  // what kda_fwd runs
};

// Which kernels kda_fwd runs (the rule is stated with KDA_FUSED_MIN_PAIRS).
// Segmented single pass without a flag: at most KDA_SEGMENTED_MAX_PAIRS pairs (two
// segments per pair still fit one round of workgroups on the compute units) and
// sequences of at least KDA_SEGMENTED_MIN_AVG_CHUNKS chunks on average, or of
// KDA_SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS up to KDA_SEGMENTED_FEW_PAIRS pairs.
bool seg_worth(const kda_desc_t *d, int64_t n_c_max)
{
    const int64_t pairs = d->num_seqs * (int64_t)d->num_heads;
    const int64_t min_avg =
        pairs <= KDA_SEGMENTED_FEW_PAIRS ? KDA_SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS : KDA_SEGMENTED_MIN_AVG_CHUNKS;
    return pairs <= KDA_SEGMENTED_MAX_PAIRS && n_c_max >= min_avg * d->num_seqs;
}

Path pick_path(const kda_desc_t *d, bool f32_path, int64_t T_tot, int64_t n_c_max)
{
    if (d->flags & KDA_FLAG_RECURRENT) return kRecurrent;
    if (d->flags & KDA_FLAG_FUSED) return kFused;
    if (d->flags & KDA_FLAG_SEGMENTED) return kSeg;
    if (d->flags & (KDA_FLAG_SPLIT | KDA_FLAG_BF16_RESIDENT_STATE)) return kSplit;
    if (T_tot <= (int64_t)KDA_RECURRENT_MAX_AVG_TOKENS * d->num_seqs) return kRecurrent;
    if (f32_path) return kSplit;
    if (seg_worth(d, n_c_max)) return kSeg;
    if (d->num_seqs * (int64_t)d->num_heads >= KDA_FUSED_MIN_PAIRS ||
        n_c_max <= (int64_t)KDA_FUSED_MAX_AVG_CHUNKS * d->num_seqs)
        return kFused;
    return kSplit;
}

// Shape-level checks shared by the size query and the forward call.
kda_status_t check_desc(const kda_desc_t *d, bool varlen, Shape *out)
{
    if (!d) return KDA_ERR_NULL_ARG;
    if (d->head_dim != KDA_HEAD_DIM || d->num_heads < 1 || d->num_heads > 65535 || d->batch < 1 ||
        d->seqlen < 0 || d->num_seqs < 1)
        return KDA_ERR_BAD_SHAPE;
    if ((d->io_dtype != KDA_DTYPE_BF16 && d->io_dtype != KDA_DTYPE_FP32) ||
        (d->state_dtype != KDA_DTYPE_BF16 && d->state_dtype != KDA_DTYPE_FP32))
        return KDA_ERR_BAD_DTYPE;
    const uint32_t known = KDA_FLAG_FP32_COMPUTE | KDA_FLAG_SPLIT | KDA_FLAG_FUSED | KDA_FLAG_RECURRENT |
                           KDA_FLAG_SCALAR_GATE | KDA_FLAG_BF16_RESIDENT_STATE | KDA_FLAG_SEGMENTED;
    if (d->flags & ~known) return KDA_ERR_BAD_ARG;
    const bool f32_path = d->io_dtype == KDA_DTYPE_FP32 || (d->flags & KDA_FLAG_FP32_COMPUTE);
    const uint32_t paths = d->flags & (KDA_FLAG_SPLIT | KDA_FLAG_FUSED | KDA_FLAG_RECURRENT | KDA_FLAG_SEGMENTED);
    if (paths & (paths - 1)) return KDA_ERR_BAD_ARG;  // more than one path flag
    if ((d->flags & (KDA_FLAG_FUSED | KDA_FLAG_SEGMENTED)) && f32_path) return KDA_ERR_BAD_ARG;
    if ((d->flags & KDA_FLAG_BF16_RESIDENT_STATE) && (f32_path || (paths & ~(uint32_t)KDA_FLAG_SPLIT)))
        return KDA_ERR_BAD_ARG;
    int64_t T_tot, n_c_max;
    const int64_t lim = (int64_t)1 << 30;  // tokens and sequences addressed with int32 on the device
    if (varlen) {
        if (d->batch != 1) return KDA_ERR_BAD_SEQLENS;
        if (d->seqlen >= lim || d->num_seqs >= lim) return KDA_ERR_BAD_SHAPE;
        T_tot = d->seqlen;
        n_c_max = (T_tot + (int64_t)(KDA_CHUNK - 1) * d->num_seqs) / KDA_CHUNK;
    } else {
        if (d->num_seqs != d->batch) return KDA_ERR_BAD_SHAPE;
        if (d->batch >= lim || d->seqlen >= lim || d->batch * d->seqlen >= lim) return KDA_ERR_BAD_SHAPE;
        T_tot = d->batch * d->seqlen;
        n_c_max = d->batch * ((d->seqlen + KDA_CHUNK - 1) / KDA_CHUNK);
    }
    if (n_c_max * (int64_t)d->num_heads >= ((int64_t)1 << 31)) return KDA_ERR_BAD_SHAPE;
    if (d->num_seqs * (int64_t)d->num_heads >= ((int64_t)1 << 31)) return KDA_ERR_BAD_SHAPE;
    out->T_tot = T_tot;
    out->n_c_max = n_c_max;
    out->f32_path = f32_path;
    out->path = pick_path(d, f32_path, T_tot, n_c_max);
    return KDA_OK;
}

}  // namespace

extern "C" size_t kda_fwd_workspace_size(const kda_desc_t *desc)
{
    // Whether cu_seqlens will be passed is not part of the description, so
    // take the larger bound over the readings the description allows.
    size_t best = 0;
    for (int varlen = 0; varlen < 2; ++varlen) {
        Shape s;
        if (check_desc(desc, varlen != 0, &s) != KDA_OK) continue;
        // the single-pass and token-by-token paths need no units, but without
        // their flags the same description is also valid for the two-stage
        // entry points
        const bool units = !(desc->flags & (KDA_FLAG_FUSED | KDA_FLAG_RECURRENT | KDA_FLAG_SEGMENTED));
        const bool look = units && kda::use_lookahead(desc->num_seqs, desc->num_heads, s.f32_path,
                                                       (desc->flags & KDA_FLAG_BF16_RESIDENT_STATE) != 0);
        size_t b = kda::ws_layout(desc->num_seqs, desc->num_heads, units ? s.n_c_max : 0, s.f32_path, look).total;
        if (s.path == kFused) {
            const size_t bf = kda::ws_layout_fused(desc->num_seqs, desc->num_heads).total;
            if (bf > b) b = bf;
        }
        if (s.path == kSeg) {
            const size_t bs = kda::ws_layout_seg(desc->num_seqs, desc->num_heads, s.n_c_max).total;
            if (bs > b) b = bs;
        }
        if (b > best) best = b;
    }
    return best;
}

namespace {

enum Stage { kPrepare = 1, kRecur = 2, kSegStage = 4 };  // kSegStage: the segmented path's stages

kda_status_t run(const void *q, const void *k, const void *v, const void *g_raw, const void *beta_raw,
                 const int32_t *cu_seqlens, const void *initial_state, void *out, void *final_state,
                 float lower_bound, const kda_desc_t *desc, void *workspace, size_t workspace_bytes,
                 void *stream, int stages)
{
    Shape s;
    const bool varlen = cu_seqlens != nullptr;
    const bool seg_stage = (stages & kSegStage) != 0;
    stages &= kPrepare | kRecur;
    kda_status_t st = check_desc(desc, varlen, &s);
    if (st != KDA_OK) return st;
    if (seg_stage) {
        if (s.f32_path || (desc->flags & (KDA_FLAG_SPLIT | KDA_FLAG_FUSED | KDA_FLAG_RECURRENT |
                                          KDA_FLAG_BF16_RESIDENT_STATE)))
            return KDA_ERR_BAD_ARG;
    } else if (stages != (kPrepare | kRecur) &&
               (desc->flags & (KDA_FLAG_FUSED | KDA_FLAG_RECURRENT | KDA_FLAG_SEGMENTED))) {
        return KDA_ERR_BAD_ARG;
    }
    const Path path = seg_stage ? kSeg : stages == (kPrepare | kRecur) ? s.path : kSplit;
    const bool no_units = path != kSplit;
    if (!isfinite(lower_bound) || lower_bound < KDA_LOWER_BOUND_MIN || lower_bound > KDA_LOWER_BOUND_MAX)
        return KDA_ERR_BAD_ARG;
    if (!isfinite(desc->scale) || !(desc->scale > 0.f)) return KDA_ERR_BAD_ARG;
    if ((desc->flags & KDA_FLAG_BF16_RESIDENT_STATE) && lower_bound > KDA_BF16_RESIDENT_MAX_LOWER_BOUND)
        return KDA_ERR_BAD_ARG;

    const int64_t H = desc->num_heads, N = desc->num_seqs;
    const size_t esz = desc->io_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t ssz = desc->state_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t tens = (size_t)s.T_tot * H * KDA_HEAD_DIM * esz;
    const size_t bet = (size_t)s.T_tot * H * esz;
    const bool sgate = (desc->flags & KDA_FLAG_SCALAR_GATE) != 0;
    const size_t gsz = sgate ? bet : tens;
    const size_t sts = (size_t)N * H * KDA_HEAD_DIM * KDA_HEAD_DIM * ssz;

    if (s.T_tot > 0 && (!q || !k || !v || !g_raw || !beta_raw || !out)) return KDA_ERR_NULL_ARG;
    if (!workspace) return KDA_ERR_WORKSPACE;
    const bool look =
        !no_units && kda::use_lookahead(N, H, s.f32_path, (desc->flags & KDA_FLAG_BF16_RESIDENT_STATE) != 0);
    const WsLayout lay = path == kSeg     ? kda::ws_layout_seg(N, H, s.n_c_max)
                         : path == kFused ? kda::ws_layout_fused(N, H)
                                          : kda::ws_layout(N, H, no_units ? 0 : s.n_c_max, s.f32_path, look);
    if (workspace_bytes < lay.total || !aligned(workspace, KDA_WORKSPACE_ALIGN)) return KDA_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g_raw, sgate ? esz : 16) ||
        !aligned(out, 16) || !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(beta_raw, esz))
        return KDA_ERR_MISALIGNED;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_ERR_MISALIGNED;

    // Overlap rules: out and the workspace touch nothing else; final_state may
    // only coincide exactly with initial_state.
    const Range rq = range_of(q, tens), rk = range_of(k, tens), rv = range_of(v, tens), rg = range_of(g_raw, gsz);
    const Range rb = range_of(beta_raw, bet), ro = range_of(out, tens);
    const Range r0 = range_of(initial_state, sts), r1 = range_of(final_state, sts);
    const Range rw = range_of(workspace, lay.total);
    const Range rc = range_of(cu_seqlens, varlen ? sizeof(int32_t) * (size_t)(N + 1) : 0);
    const Range others[] = {rq, rk, rv, rg, rb, rc};
    for (const Range &r : others)
        if (overlap(ro, r) || overlap(rw, r) || overlap(r1, r)) return KDA_ERR_BAD_ARG;
    if (overlap(ro, r0) || overlap(rw, r0) || overlap(ro, rw) || overlap(ro, r1) || overlap(rw, r1))
        return KDA_ERR_BAD_ARG;
    if (overlap(r0, r1) && r0.lo != r1.lo) return KDA_ERR_BAD_ARG;  // equal sizes: same base = same buffer

    Problem p;
    p.q = q; p.k = k; p.v = v; p.g = g_raw; p.beta = beta_raw;
    p.cu = cu_seqlens; p.s0 = initial_state; p.out = out; p.s1 = final_state;
    p.lb = lower_bound; p.scale = desc->scale;
    p.B = desc->batch; p.T = desc->seqlen; p.N = N; p.T_tot = s.T_tot; p.n_c_max = s.n_c_max;
    p.H = (int)H;
    p.io_bf16 = desc->io_dtype == KDA_DTYPE_BF16;
    p.st_bf16 = desc->state_dtype == KDA_DTYPE_BF16;
    p.f32_path = s.f32_path;
    p.scalar_gate = sgate;
    p.bf16_resident = (desc->flags & KDA_FLAG_BF16_RESIDENT_STATE) != 0;
    p.ws = static_cast<char *>(workspace);
    p.lay = lay;

    // every launch of the path (both stages, whichever the call runs) within the
    // grid limits, or nothing is enqueued
    const bool fits = path == kSeg     ? kda::fits_fused(p, true) && kda::fits_seg_finish(p)
                      : path == kFused ? kda::fits_fused(p, false)
                      : path == kRecurrent ? kda::fits_recurrent(p)
                      : p.f32_path         ? kda::fits_ref(p)
                                           : kda::fits_split(p);
    if (!fits) return KDA_ERR_BAD_SHAPE;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (path == kSeg) {
        if (stages & kPrepare) {
            if (kda::launch_chunk_map(p, hs) != hipSuccess) return KDA_ERR_HIP;
            if (s.T_tot > 0 && kda::launch_fused_seg(p, hs) != hipSuccess) return KDA_ERR_HIP;
        }
        if ((stages & kRecur) && kda::launch_seg_finish(p, hs) != hipSuccess) return KDA_ERR_HIP;
        return KDA_OK;
    }
    if (path == kFused || path == kRecurrent) {
        if (kda::launch_chunk_map(p, hs) != hipSuccess) return KDA_ERR_HIP;
        if ((path == kFused ? kda::launch_fused(p, hs) : kda::launch_recurrent(p, hs)) != hipSuccess)
            return KDA_ERR_HIP;
        return KDA_OK;
    }
    if (stages & kPrepare) {
        if (kda::launch_chunk_map(p, hs) != hipSuccess) return KDA_ERR_HIP;
        if ((p.f32_path ? kda::launch_prep_ref(p, hs) : kda::launch_prep_mfma(p, hs)) != hipSuccess)
            return KDA_ERR_HIP;
    }
    if (stages & kRecur) {
        if ((p.f32_path ? kda::launch_recur_ref(p, hs) : kda::launch_recur_mfma(p, hs)) != hipSuccess)
            return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // namespace

#define KDA_ARGS                                                                                          \
    const void *q, const void *k, const void *v, const void *g_raw, const void *beta_raw,                  \
        const int32_t *cu_seqlens, const void *initial_state, void *out, void *final_state, float lower_bound, \
        const kda_desc_t *desc, void *workspace, size_t workspace_bytes, void *stream
#define KDA_PASS                                                                                          \
    q, k, v, g_raw, beta_raw, cu_seqlens, initial_state, out, final_state, lower_bound, desc, workspace,    \
        workspace_bytes, stream

extern "C" kda_status_t kda_fwd(KDA_ARGS) { return run(KDA_PASS, kPrepare | kRecur); }
extern "C" kda_status_t kda_fwd_prepare(KDA_ARGS) { return run(KDA_PASS, kPrepare); }
extern "C" kda_status_t kda_fwd_recur(KDA_ARGS) { return run(KDA_PASS, kRecur); }
extern "C" kda_status_t kda_fwd_seg_pass(KDA_ARGS) { return run(KDA_PASS, kSegStage | kPrepare); }
extern "C" kda_status_t kda_fwd_seg_finish(KDA_ARGS) { return run(KDA_PASS, kSegStage | kRecur); }

// Scratch of kda_fwd_noalloc: the single pass's and the token-by-token path's
// workspace (chunk map and sequence order), one copy per GPU. Host code never
// passes this name to a kernel (on the host it stands for no device address);
// it uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;

// address of the current device's scratch, looked up on the first call with that
// device current and kept
hipError_t scratch_for_current_device(void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g_raw,
                                        const void *beta_raw, const int32_t *cu_seqlens,
                                        const void *initial_state, void *out, void *final_state,
                                        float lower_bound, const kda_desc_t *desc, void *stream)
{
    Shape s;
    const kda_status_t st = check_desc(desc, cu_seqlens != nullptr, &s);
    if (st != KDA_OK) return st;
    if (desc->flags & (KDA_FLAG_SPLIT | KDA_FLAG_SEGMENTED | KDA_FLAG_BF16_RESIDENT_STATE)) return KDA_ERR_BAD_ARG;
    // the paths with a small workspace: token by token where kda_fwd would take it or
    // for fp32 compute, the single pass otherwise
    kda_desc_t d = *desc;
    if (!(d.flags & (KDA_FLAG_FUSED | KDA_FLAG_RECURRENT)))
        d.flags |= (s.path == kRecurrent || s.f32_path) ? KDA_FLAG_RECURRENT : KDA_FLAG_FUSED;
    if (d.num_seqs > KDA_NOALLOC_MAX_SEQS) return KDA_ERR_TOO_LARGE;
    const size_t need = (d.flags & KDA_FLAG_FUSED) ? kda::ws_layout_fused(d.num_seqs, d.num_heads).total
                                                   : kda::ws_layout(d.num_seqs, d.num_heads, 0, s.f32_path, false).total;
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (scratch_for_current_device(&ws) != hipSuccess) return KDA_ERR_HIP;
    return run(q, k, v, g_raw, beta_raw, cu_seqlens, initial_state, out, final_state, lower_bound, &d, ws,
               KDA_NOALLOC_SCRATCH_BYTES, stream, kPrepare | kRecur);
}

extern "C" const char *kda_status_str(kda_status_t status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "bad shape (head_dim must be 128; 1 <= H <= 65535; B, N >= 1; T >= 0; sizes in range)";
    case KDA_ERR_BAD_DTYPE: return "unknown dtype code";
    case KDA_ERR_BAD_SEQLENS: return "cu_seqlens requires batch == 1";
    case KDA_ERR_BAD_ARG: return "bad argument (lower_bound, scale, unknown or conflicting flags, or overlapping buffers)";
    case KDA_ERR_WORKSPACE: return "workspace missing, too small or not 128-byte aligned";
    case KDA_ERR_MISALIGNED: return "a tensor base address is not 16-byte aligned";
    case KDA_ERR_HIP: return "HIP kernel launch failed";
    case KDA_ERR_TOO_LARGE: return "too many sequences for the static scratch of kda_fwd_noalloc";
    }
    return "unknown status";
}

extern "C" int kda_version(void) { return kVersion; }
