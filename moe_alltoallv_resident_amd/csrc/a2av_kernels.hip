// gfx950 (MI355X) kernels of the dispatch/combine path.
//
// The path follows the pages' mixture-of-experts layer (abhik.ai "Collective
// Communication for 100k+ GPUs", section "Inference: small messages, unknown sizes",
// Figure 13; qiguanping.github.io "NCCLX", section 7, figures 13-18):
//   plan      histogram of (rank, expert) and the scans that turn it into send and
//             receive offsets, all on the device (the GPU-resident metadata);
//   pack      token rows copied into expert-sorted send segments;
//   exchange  segments copied into the receiving ranks' buffers at device-computed
//             offsets (the all-to-allv), and the same kernel reversed for the return;
//   combine   gate-weighted sum of each token's k returned rows, float32 accumulate.
// Everything but the planning kernel is a row copy or a row gather, bound by HBM
// bandwidth: rows move as 16-byte vectors, one 64-lane wavefront per row, with all of
// a row's loads issued before its stores.  Nothing here is a dense contraction, so no
// matrix-core instruction is used.
#include "a2av_internal.h"

#include <algorithm>

namespace a2av {
namespace {

constexpr int kWave = 64;
constexpr int kRowsPerBlock = 4;     // 256-thread blocks, one wavefront per row
constexpr int kBlock = kWave * kRowsPerBlock;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int B> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int y = __shfl_up(v, d, kWave);
        if (lane >= d) v += y;
    }
    return v;
}

__device__ __forceinline__ int32_t load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix sum of a[0..n) in LDS, in place, by the whole block; returns the
// total to every thread.  `wsum` holds one int per wavefront plus one.
__device__ int block_exclusive_scan(int* a, int n, int* wsum) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = lane_id(), w = tid / kWave, nw = nt / kWave;
    const int per = (n + nt - 1) / nt;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += a[i];
    int incl = wave_inclusive_scan(local);
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < nw; ++i) { int c = wsum[i]; wsum[i] = run; run += c; }
        wsum[nw] = run;
    }
    __syncthreads();
    int run = wsum[w] + incl - local;
    for (int i = lo; i < hi; ++i) { int c = a[i]; a[i] = run; run += c; }
    int total = wsum[nw];
    __syncthreads();
    return total;
}

// Receive side of the metadata exchange, run by the last block of a planning grid once
// every sender has published its column recv_counts[.][s]: for every destination d,
// recv_off[d][s] = sum over s' < s of recv_counts[d][s'] (one wavefront per d).
__device__ void finish_recv_tables(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status) {
    const int R = sh.R, lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
    for (int d = w; d < R; d += nw) {
        int carry = 0;
        for (int s0 = 0; s0 < R; s0 += kWave) {
            const int s = s0 + lane;
            const int c = s < R ? load_agent(tb.recv_counts + (int64_t)d * R + s) : 0;
            const int incl = wave_inclusive_scan(c);
            if (s < R) {
                const int off = carry + incl - c;
                tb.recv_off[(int64_t)d * (R + 1) + s] = off;
                if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + s] = off;
                if (out.recv_counts) out.recv_counts[(int64_t)d * R + s] = c;
            }
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) {
            tb.recv_off[(int64_t)d * (R + 1) + R] = carry;
            if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + R] = carry;
            if ((int64_t)carry > sh.cap) atomicOr(status, 2u);
        }
    }
}

// Arrival ticket: returns true in exactly one block, the last to arrive, after all
// blocks' earlier global writes are visible to it.  The last block resets the ticket
// so the next launch (or graph replay) starts from zero.
__device__ bool last_block_arrives(uint32_t* ticket, int* flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        *flag = (prev == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!*flag) return false;
    __threadfence();
    return true;
}

// ------------------------------------------------------------------------------------
// plan: one block per rank (histogram, scans, stable positions), then the last block
// forms every rank's receive offsets.
//
// Positions are a stable counting sort by (expert, token, slot).  Each wavefront owns a
// contiguous run of the rank's assignments and walks it 64 at a time.  Lanes holding
// the same expert find each other with one ballot per bit of the expert id (the AND of
// the matching ballots is the set of lanes with an equal id); a lane's rank among them
// is the popcount of that set below it.  The lowest such lane adds the group size to
// the wavefront's private LDS counter for that expert, so no atomics are needed and the
// result does not depend on timing.  Counters of all wavefronts are then scanned in
// (expert, wavefront) order into final bases.
// ------------------------------------------------------------------------------------
struct PlanArgs {
    Shape sh;
    Tables tb;
    Outputs out;
    const int32_t* ids;
    uint32_t* status;
};

__global__ void __launch_bounds__(1024) plan_kernel(PlanArgs a) {
    extern __shared__ int lds[];
    __shared__ int wsum[17];
    __shared__ int flag;
    const Shape& sh = a.sh;
    const int E = sh.E, R = sh.R;
    const int tid = threadIdx.x, nt = blockDim.x, lane = lane_id(), w = tid / kWave, nw = nt / kWave;
    const int s = blockIdx.x;
    int* cw = lds;               // [nw][E] per-wavefront counters, later bases
    int* tot = lds + nw * E;     // [E] per-expert totals, later exclusive offsets

    for (int i = tid; i < nw * E; i += nt) cw[i] = 0;
    __syncthreads();

    const int64_t TK = sh.TK;
    const int32_t* ids = a.ids + (int64_t)s * TK;
    int32_t* pos = a.tb.pos + (int64_t)s * TK;
    const int64_t chunk = ((TK + nw - 1) / nw + kWave - 1) / kWave * kWave;
    const int64_t a0 = min(TK, (int64_t)w * chunk), a1 = min(TK, a0 + chunk);
    int* mine = cw + w * E;
    bool bad = false;

    // pass 1: rank of every assignment among equal experts inside its wavefront's run
    for (int64_t base = a0; base < a1; base += kWave) {
        const int64_t i = base + lane;
        const bool valid = i < a1;
        const int e = valid ? ids[i] : 0;
        const bool in = valid && e >= 0 && e < E;
        bad |= valid && !in;
        uint64_t match = __ballot(in);
        for (int b = 0; b < sh.nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(in && bit);
            match &= bit ? m : ~m;
        }
        if (in) {
            const int r = __popcll(match & lanes_below(lane));
            const int c = mine[e];
            pos[i] = c + r;
            if (r == 0) mine[e] = c + __popcll(match);
        }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(a.status, 1u);
    __syncthreads();

    // per expert: wavefront bases (exclusive over wavefronts) and the rank's count
    for (int e = tid; e < E; e += nt) {
        int run = 0;
        for (int v = 0; v < nw; ++v) { const int c = cw[v * E + e]; cw[v * E + e] = run; run += c; }
        tot[e] = run;
        a.tb.cnt[(int64_t)s * E + e] = run;
        if (a.out.split) a.out.split[(int64_t)s * E + e] = run;
    }
    __syncthreads();
    const int total = block_exclusive_scan(tot, E, wsum);   // tot[e] = first row of expert e

    // send segments: destination d holds experts d*epr .. d*epr+epr-1, which are
    // consecutive in the sorted order
    for (int d = tid; d <= R; d += nt) {
        const int lo = d < R ? tot[d * sh.epr] : total;
        a.tb.send_off[(int64_t)s * (R + 1) + d] = lo;
        if (d < R) {
            const int hi = d + 1 < R ? tot[(d + 1) * sh.epr] : total;
            store_agent(a.tb.recv_counts + (int64_t)d * R + s, hi - lo);   // column s of [dst][src]
        }
    }
    for (int i = tid; i < nw * E; i += nt) cw[i] += tot[i % E];
    __syncthreads();

    // pass 2: final positions
    for (int64_t base = a0; base < a1; base += kWave) {
        const int64_t i = base + lane;
        if (i < a1) {
            const int e = ids[i];
            pos[i] = (e >= 0 && e < E) ? mine[e] + pos[i] : -1;
        }
    }

    if (!last_block_arrives(a.tb.ticket, &flag)) return;
    finish_recv_tables(sh, a.tb, a.out, a.status);
    if (tid == 0) __hip_atomic_store(a.tb.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The bare collective's planning: send offsets from caller counts, one block per sender.
struct CountsArgs {
    Shape sh;
    Tables tb;
    Outputs out;
    const int32_t* send_counts;
    uint32_t* status;
};

__global__ void __launch_bounds__(256) plan_from_counts_kernel(CountsArgs a) {
    __shared__ int sc[kMaxRanks + 1];
    __shared__ int wsum[5];
    __shared__ int flag;
    const int R = a.sh.R, tid = threadIdx.x, nt = blockDim.x, s = blockIdx.x;
    for (int d = tid; d < R; d += nt) sc[d] = a.send_counts[(int64_t)s * R + d];
    __syncthreads();
    if (tid == 0) {
        int64_t sum = 0;
        bool ok = true;
        for (int d = 0; d < R; ++d) { ok &= sc[d] >= 0; sum += sc[d]; }
        flag = ok && sum <= a.sh.TK;
        if (!flag) atomicOr(a.status, 1u);
    }
    __syncthreads();
    if (!flag)
        for (int d = tid; d < R; d += nt) sc[d] = 0;
    __syncthreads();
    const int total = block_exclusive_scan(sc, R, wsum);
    for (int d = tid; d <= R; d += nt) {
        const int lo = d < R ? sc[d] : total;
        a.tb.send_off[(int64_t)s * (R + 1) + d] = lo;
        if (d < R) {
            const int hi = d + 1 < R ? sc[d + 1] : total;
            store_agent(a.tb.recv_counts + (int64_t)d * R + s, hi - lo);
        }
    }
    if (!last_block_arrives(a.tb.ticket, &flag)) return;
    finish_recv_tables(a.sh, a.tb, a.out, a.status);
    if (tid == 0) __hip_atomic_store(a.tb.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------
// Row movement.  One wavefront per row; lane l moves vectors l, l+64, ...; U vectors
// per lane are loaded before any is stored, so a 10 KiB row is in flight at once.
// ------------------------------------------------------------------------------------
template <typename V, int U>
__device__ __forceinline__ void copy_row(V* __restrict__ dst, const V* __restrict__ src, int nvec, int lane) {
    for (int base = 0; base < nvec; base += kWave * U) {
        V r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < nvec) r[u] = src[v];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < nvec) dst[v] = r[u];
        }
    }
}

template <typename V>
__device__ __forceinline__ void zero_row(V* __restrict__ dst, int nvec, int lane) {
    for (int v = lane; v < nvec; v += kWave) dst[v] = V{};
}

// Which destination segment holds send row p of a sender: the number of segment ends
// send_off[d+1] at or below p (one ballot per 64 destinations).
__device__ __forceinline__ int segment_of(const int32_t* so, int R, int64_t p, int lane) {
    int d = 0;
    for (int c0 = 0; c0 < R; c0 += kWave) {
        const int i = c0 + lane;
        d += __popcll(__ballot(i < R && (int64_t)so[i + 1] <= p));
    }
    return d;
}

// pack: row x[s][t] to its k places in s's send buffer.
template <typename V, int U>
__global__ void __launch_bounds__(kBlock) pack_kernel(const V* __restrict__ x, V* __restrict__ send,
                                                      const int32_t* __restrict__ pos, Shape sh, int nvec) {
    const int lane = lane_id();
    const int64_t n = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (n >= (int64_t)sh.R * sh.T) return;
    const int64_t s = n / sh.T;
    const int k = sh.k;
    const int my = lane < k ? pos[n * k + lane] : -1;
    const V* src = x + n * nvec;
    V* seg = send + s * sh.TK * nvec;
    for (int base = 0; base < nvec; base += kWave * U) {
        V r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < nvec) r[u] = src[v];
        }
        for (int j = 0; j < k; ++j) {
            const int pj = __builtin_amdgcn_readlane(my, j);
            if (pj < 0 || pj >= sh.TK) continue;      // dropped slot (never out of the send buffer)
            V* dst = seg + (int64_t)pj * nvec;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * kWave + lane;
                if (v < nvec) dst[v] = r[u];
            }
        }
    }
}

// exchange: send row (s, p) <-> receive row (d, q).  Forward copies send -> recv and
// drops rows past the capacity; reverse copies recv-layout expert outputs back to the
// send places and writes zeros where a row was dropped.
template <typename V, int U, bool REVERSE>
__global__ void __launch_bounds__(kBlock) exchange_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                          const int32_t* __restrict__ send_off,
                                                          const int32_t* __restrict__ recv_off, Shape sh, int nvec) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (g >= (int64_t)sh.R * sh.TK) return;
    const int R = sh.R;
    const int64_t s = g / sh.TK, p = g - s * sh.TK;
    const int32_t* so = send_off + s * (R + 1);
    if (p >= so[R]) return;
    const int d = segment_of(so, R, p, lane);
    const int64_t q = (int64_t)recv_off[(int64_t)d * (R + 1) + s] + (p - so[d]);
    const int64_t send_row = s * sh.TK + p, recv_row = (int64_t)d * sh.cap + q;
    const bool in_cap = q >= 0 && q < sh.cap;
    if (!REVERSE) {
        if (!in_cap) return;
        copy_row<V, U>(dst + recv_row * nvec, src + send_row * nvec, nvec, lane);
    } else {
        if (!in_cap) { zero_row<V>(dst + send_row * nvec, nvec, lane); return; }
        copy_row<V, U>(dst + send_row * nvec, src + recv_row * nvec, nvec, lane);
    }
}

// ---- element access for the arithmetic kernels --------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int B> struct Words;   // a vector seen as 32-bit words
template <> struct Words<16> {
    __device__ static uint32_t get(const u32x4& v, int i) { return v[i]; }
    __device__ static void set(u32x4& v, int i, uint32_t x) { v[i] = x; }
};
template <> struct Words<8> {
    __device__ static uint32_t get(const u32x2& v, int i) { return v[i]; }
    __device__ static void set(u32x2& v, int i, uint32_t x) { v[i] = x; }
};
template <> struct Words<4> {
    __device__ static uint32_t get(const uint32_t& v, int) { return v; }
    __device__ static void set(uint32_t& v, int, uint32_t x) { v = x; }
};

// Elements per vector and their float values.
template <int B, int DT> struct Elems {
    static constexpr int N = DT == 1 ? B / 2 : B / 4;
    using V = typename Vec<B>::T;
    __device__ static float get(const V& v, int i) {
        if constexpr (B == 2) {
            return __uint_as_float((uint32_t)v << 16);
        } else if constexpr (DT == 1) {
            const uint32_t w = Words<B>::get(v, i / 2);
            return (i & 1) ? bf16_hi(w) : bf16_lo(w);
        } else {
            return __uint_as_float(Words<B>::get(v, i));
        }
    }
    __device__ static V pack(const float* f) {
        V v{};
        if constexpr (B == 2) {
            v = (uint16_t)to_bf16(f[0]);
        } else if constexpr (DT == 1) {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) Words<B>::set(v, i, to_bf16(f[2 * i]) | (to_bf16(f[2 * i + 1]) << 16));
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) Words<B>::set(v, i, __float_as_uint(f[i]));
        }
        return v;
    }
};

// combine: y[s][t] = round(sum_j g_j * ret_s[pos_j]) with one float32 FMA per slot in
// slot order, starting from 0.
template <int B, int DT, int U>
__global__ void __launch_bounds__(kBlock) combine_kernel(const typename Vec<B>::T* __restrict__ ret,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ gates,
                                                         typename Vec<B>::T* __restrict__ y, Shape sh, int nvec) {
    using V = typename Vec<B>::T;
    using El = Elems<B, DT>;
    constexpr int NE = El::N;
    const int lane = lane_id();
    const int64_t n = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (n >= (int64_t)sh.R * sh.T) return;
    const int64_t s = n / sh.T;
    const int k = sh.k;
    const int my_p = lane < k ? pos[n * k + lane] : -1;
    const float my_g = lane < k ? gates[n * k + lane] : 0.0f;
    const V* seg = ret + s * sh.TK * nvec;
    V* out = y + n * nvec;
    for (int base = 0; base < nvec; base += kWave * U) {
        float acc[U][NE];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[u][e] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int pj = __builtin_amdgcn_readlane(my_p, j);
            const float gj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_g), j));
            if (pj < 0 || pj >= sh.TK) continue;      // dropped slot adds nothing
            const V* row = seg + (int64_t)pj * nvec;
            V r[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * kWave + lane;
                if (v < nvec) r[u] = row[v];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[u][e] = __builtin_fmaf(gj, El::get(r[u], e), acc[u][e]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < nvec) out[v] = El::pack(acc[u]);
        }
    }
}

// Harness expert stand-in over every received row: identity, or scale by 1 + e/256
// with one rounding (the float32 product of a bf16 value and 1 + e/256 is exact).
// Rows are found from the send side as in the exchange; the row's expert is the one
// whose slice of the sender's expert-sorted segment holds it.
template <int B, int DT, int U>
__global__ void __launch_bounds__(kBlock) expert_kernel(const typename Vec<B>::T* __restrict__ in,
                                                        typename Vec<B>::T* out,
                                                        const int32_t* __restrict__ send_off,
                                                        const int32_t* __restrict__ recv_off,
                                                        const int32_t* __restrict__ cnt, Shape sh, int nvec,
                                                        int mode) {
    using V = typename Vec<B>::T;
    using El = Elems<B, DT>;
    constexpr int NE = El::N;
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (g >= (int64_t)sh.R * sh.TK) return;
    const int R = sh.R;
    const int64_t s = g / sh.TK, p = g - s * sh.TK;
    const int32_t* so = send_off + s * (R + 1);
    if (p >= so[R]) return;
    const int d = segment_of(so, R, p, lane);
    const int64_t i = p - so[d];
    const int64_t q = (int64_t)recv_off[(int64_t)d * (R + 1) + s] + i;
    if (q < 0 || q >= sh.cap) return;
    const int64_t row = (int64_t)d * sh.cap + q;
    if (mode == 0) {
        if (in != out) copy_row<V, U>(out + row * nvec, in + row * nvec, nvec, lane);
        return;
    }
    // local expert: number of the sender's per-expert counts for d whose running
    // sum is at or below i
    const int32_t* c = cnt + s * sh.E + (int64_t)d * sh.epr;
    int le = 0, carry = 0;
    for (int c0 = 0; c0 < sh.epr; c0 += kWave) {
        const int idx = c0 + lane;
        const int v = idx < sh.epr ? c[idx] : 0;
        const int incl = carry + wave_inclusive_scan(v);
        le += __popcll(__ballot(idx < sh.epr && (int64_t)incl <= i));
        carry = __shfl(incl, kWave - 1, kWave);
    }
    const float scale = 1.0f + (float)(d * sh.epr + le) / 256.0f;
    const V* src = in + row * nvec;
    V* dst = out + row * nvec;
    for (int v = lane; v < nvec; v += kWave) {
        const V r = src[v];
        float f[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) f[e] = El::get(r, e) * scale;
        dst[v] = El::pack(f);
    }
}

__global__ void __launch_bounds__(1024) route_step_kernel(const int32_t* __restrict__ ids_table,
                                                          const float* __restrict__ gates_table, int32_t steps,
                                                          int64_t n, int32_t* counter, int32_t* __restrict__ ids,
                                                          float* __restrict__ gates) {
    const int32_t c = *counter;
    const int64_t step = ((int64_t)c % steps + steps) % steps;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        ids[i] = ids_table[step * n + i];
        gates[i] = gates_table[step * n + i];
    }
    __syncthreads();
    if (threadIdx.x == 0) *counter = c + 1;
}

// ---- launch helpers ------------------------------------------------------------------
inline unsigned row_blocks(int64_t rows) { return (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock); }

// Vectors per lane kept in flight: the smallest of 1, 2, 4, 8, 16 covering a row.
template <typename F>
hipError_t with_unroll(int nvec, F&& f) {
    const int per_lane = (nvec + kWave - 1) / kWave;
    if (per_lane <= 1) return f(std::integral_constant<int, 1>{});
    if (per_lane <= 2) return f(std::integral_constant<int, 2>{});
    if (per_lane <= 4) return f(std::integral_constant<int, 4>{});
    if (per_lane <= 8) return f(std::integral_constant<int, 8>{});
    return f(std::integral_constant<int, 16>{});
}

template <typename F>
hipError_t with_vec(int vec, F&& f) {
    switch (vec) {
        case 16: return f(std::integral_constant<int, 16>{});
        case 8: return f(std::integral_constant<int, 8>{});
        case 4: return f(std::integral_constant<int, 4>{});
        default: return f(std::integral_constant<int, 2>{});
    }
}

}  // namespace

int pick_vec_bytes(int64_t row_bytes, const void* const* ptrs, int nptrs) {
    for (int v : {16, 8, 4, 2}) {
        bool ok = row_bytes % v == 0;
        for (int i = 0; i < nptrs && ok; ++i) ok = ((uintptr_t)ptrs[i] % v) == 0;
        if (ok) return v;
    }
    return 0;
}

hipError_t launch_plan(const Shape& sh, const Tables& tb, const int32_t* ids, const Outputs& out,
                       uint32_t* status, hipStream_t st) {
    // wavefronts per block: as many as fit (nw + 1) * E counters in 63 KiB (the
    // kernel's static LDS takes the rest of 64 KiB), at most 16
    const int nw = std::max(1, std::min(16, (int)(kPlanLdsBytes / (4 * (int64_t)sh.E)) - 1));
    const size_t lds = (size_t)(nw + 1) * sh.E * sizeof(int);
    PlanArgs a{sh, tb, out, ids, status};
    hipLaunchKernelGGL(plan_kernel, dim3(sh.R), dim3(nw * kWave), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_plan_from_counts(const Shape& sh, const Tables& tb, const int32_t* send_counts,
                                   const Outputs& out, uint32_t* status, hipStream_t st) {
    CountsArgs a{sh, tb, out, send_counts, status};
    hipLaunchKernelGGL(plan_from_counts_kernel, dim3(sh.R), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_pack(const Shape& sh, const Tables& tb, const void* x, void* send, int vec, hipStream_t st) {
    const int64_t N = (int64_t)sh.R * sh.T;
    if (N == 0) return hipSuccess;
    const int nvec = (int)(sh.row_bytes / vec);
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(nvec, [&](auto U) {
            hipLaunchKernelGGL((pack_kernel<V, decltype(U)::value>), dim3(row_blocks(N)), dim3(kBlock), 0, st,
                               (const V*)x, (V*)send, tb.pos, sh, nvec);
            return hipGetLastError();
        });
    });
}

hipError_t launch_exchange(const Shape& sh, const Tables& tb, const void* src, void* dst, bool reverse, int vec,
                           hipStream_t st) {
    const int64_t rows = (int64_t)sh.R * sh.TK;
    if (rows == 0) return hipSuccess;
    const int nvec = (int)(sh.row_bytes / vec);
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(nvec, [&](auto U) {
            if (reverse)
                hipLaunchKernelGGL((exchange_kernel<V, decltype(U)::value, true>), dim3(row_blocks(rows)),
                                   dim3(kBlock), 0, st, (const V*)src, (V*)dst, tb.send_off, tb.recv_off, sh, nvec);
            else
                hipLaunchKernelGGL((exchange_kernel<V, decltype(U)::value, false>), dim3(row_blocks(rows)),
                                   dim3(kBlock), 0, st, (const V*)src, (V*)dst, tb.send_off, tb.recv_off, sh, nvec);
            return hipGetLastError();
        });
    });
}

template <int B, int DT>
static hipError_t launch_combine_t(const Shape& sh, const Tables& tb, const void* ret, const float* gates, void* y,
                                   hipStream_t st) {
    using V = typename Vec<B>::T;
    const int nvec = (int)(sh.row_bytes / B);
    const int64_t N = (int64_t)sh.R * sh.T;
    return with_unroll(nvec, [&](auto U) {
        // keep float accumulators within a sane register budget
        constexpr int UU = (decltype(U)::value * Elems<B, DT>::N > 64) ? 64 / Elems<B, DT>::N : decltype(U)::value;
        hipLaunchKernelGGL((combine_kernel<B, DT, UU>), dim3(row_blocks(N)), dim3(kBlock), 0, st, (const V*)ret,
                           tb.pos, gates, (V*)y, sh, nvec);
        return hipGetLastError();
    });
}

hipError_t launch_combine(const Shape& sh, const Tables& tb, const void* ret, const float* gates, void* y, int vec,
                          hipStream_t st) {
    if ((int64_t)sh.R * sh.T == 0) return hipSuccess;
    if (sh.dtype == 1) {
        switch (vec) {
            case 16: return launch_combine_t<16, 1>(sh, tb, ret, gates, y, st);
            case 8: return launch_combine_t<8, 1>(sh, tb, ret, gates, y, st);
            case 4: return launch_combine_t<4, 1>(sh, tb, ret, gates, y, st);
            default: return launch_combine_t<2, 1>(sh, tb, ret, gates, y, st);
        }
    }
    switch (vec) {
        case 16: return launch_combine_t<16, 0>(sh, tb, ret, gates, y, st);
        case 8: return launch_combine_t<8, 0>(sh, tb, ret, gates, y, st);
        default: return launch_combine_t<4, 0>(sh, tb, ret, gates, y, st);
    }
}

template <int B, int DT>
static hipError_t launch_expert_t(const Shape& sh, const Tables& tb, const void* in, void* out, int mode,
                                  hipStream_t st) {
    using V = typename Vec<B>::T;
    const int nvec = (int)(sh.row_bytes / B);
    const int64_t rows = (int64_t)sh.R * sh.TK;
    return with_unroll(nvec, [&](auto U) {
        hipLaunchKernelGGL((expert_kernel<B, DT, decltype(U)::value>), dim3(row_blocks(rows)), dim3(kBlock), 0, st,
                           (const V*)in, (V*)out, tb.send_off, tb.recv_off, tb.cnt, sh, nvec, mode);
        return hipGetLastError();
    });
}

hipError_t launch_expert(const Shape& sh, const Tables& tb, const void* in, void* out, int mode, int vec,
                         hipStream_t st) {
    if ((int64_t)sh.R * sh.TK == 0) return hipSuccess;
    if (sh.dtype == 1) {
        switch (vec) {
            case 16: return launch_expert_t<16, 1>(sh, tb, in, out, mode, st);
            case 8: return launch_expert_t<8, 1>(sh, tb, in, out, mode, st);
            case 4: return launch_expert_t<4, 1>(sh, tb, in, out, mode, st);
            default: return launch_expert_t<2, 1>(sh, tb, in, out, mode, st);
        }
    }
    switch (vec) {
        case 16: return launch_expert_t<16, 0>(sh, tb, in, out, mode, st);
        case 8: return launch_expert_t<8, 0>(sh, tb, in, out, mode, st);
        default: return launch_expert_t<4, 0>(sh, tb, in, out, mode, st);
    }
}

hipError_t launch_route_step(const int32_t* ids_table, const float* gates_table, int32_t steps, int64_t n,
                             int32_t* counter, int32_t* ids, float* gates, hipStream_t st) {
    hipLaunchKernelGGL(route_step_kernel, dim3(1), dim3(1024), 0, st, ids_table, gates_table, steps, n, counter, ids,
                       gates);
    return hipGetLastError();
}

}  // namespace a2av
