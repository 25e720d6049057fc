// kda_internal.h -- shared definitions of the KDA forward library (not part of
// the public ABI). Workspace layout, launch parameters and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;     // head dimension K = V
constexpr int kC = 16;      // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;  // L2-norm epsilon: x / sqrt(sum x^2 + eps)

// ---------------------------------------------------------------------------
// Workspace layout.
//
//   [header 128 B] [tok_off: (N+1) int32] [chunk_off: (N+1) int32] [units]
//
// tok_off[n]  : first token of sequence n (sanitised copy of cu_seqlens).
// chunk_off[n]: first global chunk of sequence n; chunk_off[N] = chunks in use.
// A "unit" is one (chunk, head). Unit u = h * n_c_max + global_chunk holds what
// the chunk-parallel kernel hands the recurrence kernel; the chunks of one
// (sequence, head) are therefore contiguous.
//
// bf16 path unit (18944 B), every block in the lane order the recurrence
// kernel's matrix-core instructions consume (64 lanes x 16 B per 1 KB slab):
//   KB   4096  K_b  = khat * exp(G_i)           bf16, 16x16x32 A-operand order
//   QB   4096  Q_b  = s qhat * exp(G_i)         bf16, same order
//   KE   8192  K_end= khat * exp(G_last - G_i)  as a bf16 hi/lo pair, 2 KB per tile pair
//              p: lane L's 32 bytes are tile 2p's four tokens' hi values, then their lo
//              values, then tile 2p+1's (16x16x16 A-operand order for each half, so 16
//              bytes form a 16x16x32 operand [hi | lo])
//   AB   1024  (A^kk Diag(beta))^T  split into bf16 hi/lo: lane-major {hi x4, lo x4}
//   AQ   1024  (A^qk)^T             split into bf16 hi/lo: lane-major {hi x4, lo x4}
//   GM    512  gamma = exp(G_last)              fp32 [128]
// fp32 path unit (27136 B), plain row-major:
//   KB 8192 [16][128], QB 8192, KE 8192, AB 1024 [16][16] (A^kk Diag(beta)),
//   AQ 1024 [16][16] (A^qk), GM 512.
// ---------------------------------------------------------------------------
constexpr size_t kHeaderBytes = 128;

struct UnitLayout {
    size_t kb, qb, ke, ab, aq, gm, bytes;
};
constexpr UnitLayout kUnitBf16 = {0, 4096, 8192, 16384, 17408, 18432, 18944};
constexpr UnitLayout kUnitF32 = {0, 8192, 16384, 24576, 25600, 26624, 27136};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Few (sequence, head) pairs: the bf16 recurrence runs in look-ahead form, which
// also needs each chunk's K_end in K_b's order (4096 B per (chunk, head), after the
// units). Decided from the shape and flags alone, so separate stage calls agree.
constexpr int64_t kLookMaxPairs = 96;
constexpr size_t kKetBytes = 4096;
inline bool use_lookahead(int64_t N, int64_t H, bool f32_path, bool bf16_resident)
{
    return !f32_path && !bf16_resident && N * H < kLookMaxPairs;
}

// Segmented single pass (few (sequence, head) pairs, long sequences): each sequence
// is cut into G = max(2, kSegTargetGroups / pairs) segments (from the average
// sequence), so that at most about kSegTargetGroups (segment, head) workgroups, one
// per compute unit, run at once. Every segment after the first is L chunks long;
// the first is L0 = L + L/2 long, because its workgroups skip the transfer run and
// take about a third less time per chunk. Workspace after the chunk map:
//   seg_off [N+1] int32             exclusive scan of segments per sequence
//   sfin    [seg_max][H][128][128]  fp32, segment's final state from S = 0 (seg 0: S_0), in
//                                   tile order (state_tile)
//   phi     [seg_max][H][8][4][2][64][8] bf16, segment's key-space transfer Phi, transposed
//                                   and split into hi and lo halves, in the scan's
//                                   matrix-core operand order (key tile, k step, half, lane)
//   sin     [seg_max][H][128][128]  fp32, true state entering the segment, in tile order
//   ybuf    [n_c_max][H][4][64][8]  bf16, y_t = Phi_t (s qhat_t) within the segment: one
//                                   4 KB tile per (chunk, head) in the order the correction's
//                                   matrix-core operand takes it (k step, lane, 8 channels),
//                                   so each of its loads reads 1 KB in one piece
constexpr int64_t kSegTargetGroups = 256;
// Tile order of a [128][128] state in the workspace (element of value row v, key channel
// k): 16-row slice v / 16, 16-key tile k / 16, then lane 16 ((k / 4) % 4) + v % 16 and
// element k % 4, so four consecutive keys of one row are one 16-byte piece and each
// (slice, tile) block is 1 KB: the single pass's consumer lanes and the scan's
// matrix-core lanes each store or load a block in one access.
__host__ __device__ inline int state_tile(int v, int k)
{
    return (((v >> 4) * 8 + (k >> 4)) * 64 + 16 * ((k >> 2) & 3) + (v & 15)) * 4 + (k & 3);
}
constexpr int64_t kSegMinChunks = 8;
inline int64_t seg_first_for(int64_t seg_len) { return seg_len + (seg_len + 1) / 2; }
inline int64_t seg_len_for(int64_t N, int64_t H, int64_t n_c_max)
{
    const int64_t pairs = N * H;
    int64_t G = kSegTargetGroups / pairs;
    if (G < 2) G = 2;
    const int64_t avg = (n_c_max + N - 1) / N;
    // L0 + (G - 1) L = avg with L0 = 3 L / 2
    const int64_t l = (2 * avg + 2 * G) / (2 * G + 1);
    return l > kSegMinChunks ? l : kSegMinChunks;
}
// upper bound of the segment count given sum_n chunks_n <= n_c_max: every segment
// but a sequence's last holds at least L chunks
inline int64_t seg_max_for(int64_t N, int64_t n_c_max, int64_t seg_len) { return n_c_max / seg_len + N; }

// first chunk of segment g within its sequence, and the number of segments of a
// sequence of nc chunks
__host__ __device__ inline int seg_start(int g, int L, int L0) { return g == 0 ? 0 : L0 + (g - 1) * L; }
__host__ __device__ inline int seg_count(int nc, int L, int L0)
{
    return nc <= 0 ? 0 : nc <= L0 ? 1 : 1 + (nc - L0 + L - 1) / L;
}

struct WsLayout {
    size_t tok_off, chunk_off, units, unit_bytes, ket, total;
    size_t seg_off, sfin, phi, sin, ybuf;
    size_t order;  // single pass: sequences longest first, [N] int32 (0: not kept)
    int64_t n_c_max, seg_len, seg_first, seg_max;
};

inline WsLayout ws_layout(int64_t N, int64_t H, int64_t n_c_max, bool f32_path, bool lookahead)
{
    WsLayout L;
    L.tok_off = kHeaderBytes;
    L.chunk_off = align_up(L.tok_off + sizeof(int32_t) * (size_t)(N + 1), 128);
    L.units = align_up(L.chunk_off + sizeof(int32_t) * (size_t)(N + 1), 128);
    L.unit_bytes = f32_path ? kUnitF32.bytes : kUnitBf16.bytes;
    L.n_c_max = n_c_max;
    const size_t end = L.units + L.unit_bytes * (size_t)H * (size_t)n_c_max;
    L.ket = lookahead ? align_up(end, 128) : 0;
    L.total = lookahead ? L.ket + kKetBytes * (size_t)H * (size_t)n_c_max : end;
    L.seg_off = L.sfin = L.phi = L.sin = L.ybuf = 0;
    L.order = 0;
    L.seg_len = L.seg_first = L.seg_max = 0;
    return L;
}

// layout of the single pass: the chunk map and the order in which its (sequence,
// head) workgroups take the sequences, longest first, so the ragged tail of a batch
// with more workgroups than compute units is short ones
inline WsLayout ws_layout_fused(int64_t N, int64_t H)
{
    WsLayout L = ws_layout(N, H, 0, false, false);
    L.order = L.units;
    L.total = align_up(L.order + sizeof(int32_t) * (size_t)N, 128);
    return L;
}

// layout of the segmented single pass (no units)
inline WsLayout ws_layout_seg(int64_t N, int64_t H, int64_t n_c_max)
{
    WsLayout L = ws_layout(N, H, 0, false, false);
    L.n_c_max = n_c_max;
    L.seg_len = seg_len_for(N, H, n_c_max);
    L.seg_first = seg_first_for(L.seg_len);
    L.seg_max = seg_max_for(N, n_c_max, L.seg_len);
    const size_t st = (size_t)L.seg_max * (size_t)H * kD * kD * sizeof(float);
    L.seg_off = L.units;
    L.sfin = align_up(L.seg_off + sizeof(int32_t) * (size_t)(N + 1), 128);
    L.phi = L.sfin + st;
    L.sin = L.phi + st;
    L.ybuf = L.sin + st;
    L.total = L.ybuf + (size_t)n_c_max * (size_t)H * kC * kD * sizeof(uint16_t);
    return L;
}

// Everything a launch needs (device pointers and sizes, already validated).
struct Problem {
    const void *q, *k, *v, *g, *beta;
    const int32_t *cu;      // device or nullptr
    const void *s0;         // device or nullptr
    void *out, *s1;         // out device; s1 device or nullptr
    float lb, scale;
    int64_t B, T, N, T_tot, n_c_max;
    int H;
    bool io_bf16, st_bf16, f32_path;
    bool scalar_gate;       // g_raw is [T][H] (one gate per token and head), not [T][H][128]
    bool bf16_resident;     // bf16 recurrence: state rounded to bf16 between chunk updates
    char *ws;
    WsLayout lay;
};

// Launch extents: a launch keeps its work-items along x below 2^32 and its grid's y
// extent within 65535. fits_* check every launch of a path on the host, with the
// same grid arithmetic as the launches, before anything is enqueued.
inline bool grid_fits(int64_t gx, int64_t gy, int64_t threads)
{
    return gx * threads < ((int64_t)1 << 32) && gy <= 65535;
}
bool fits_split(const Problem &p);       // k1_mfma, then k2_mfma or k2_look
bool fits_ref(const Problem &p);         // k1_ref, k2_ref (and the chunk map)
bool fits_fused(const Problem &p, bool seg);
bool fits_recurrent(const Problem &p);
bool fits_seg_finish(const Problem &p);  // kseg_scan, kseg_correct

hipError_t launch_chunk_map(const Problem &p, hipStream_t s);   // K0
hipError_t launch_prep_ref(const Problem &p, hipStream_t s);    // fp32 K1
hipError_t launch_recur_ref(const Problem &p, hipStream_t s);   // fp32 K2
hipError_t launch_prep_mfma(const Problem &p, hipStream_t s);   // bf16 K1
hipError_t launch_recur_mfma(const Problem &p, hipStream_t s);  // bf16 K2
hipError_t launch_fused(const Problem &p, hipStream_t s);       // bf16 single pass
hipError_t launch_recurrent(const Problem &p, hipStream_t s);   // token-by-token (decode)
hipError_t launch_fused_seg(const Problem &p, hipStream_t s);   // bf16 segmented single pass
hipError_t launch_seg_finish(const Problem &p, hipStream_t s);  // segment scan and output correction

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld_elem(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld_elem<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t *p, int64_t i)
{
    return bf16_bits_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void st_elem(T *p, int64_t i, float x);
template <> __device__ __forceinline__ void st_elem<float>(float *p, int64_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void st_elem<uint16_t>(uint16_t *p, int64_t i, float x)
{
    p[i] = f32_to_bf16_bits(x);
}

// Sequence owning global chunk c: largest n in [0, N) with chunk_off[n] <= c.
__device__ __forceinline__ int find_seq(const int32_t *chunk_off, int N, int c)
{
    int lo = 0, hi = N;  // invariant: chunk_off[lo] <= c < chunk_off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= c) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace kda
