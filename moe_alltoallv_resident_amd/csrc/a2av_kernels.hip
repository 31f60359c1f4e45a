// gfx950 (MI355X) kernels of the dispatch/combine path.
//
// The path follows the pages' mixture-of-experts layer (abhik.ai "Collective
// Communication for 100k+ GPUs", section "Inference: small messages, unknown sizes",
// Figure 13; qiguanping.github.io "NCCLX", section 7, figures 13-18):
//   plan      per rank: histogram of (rank, expert), the scans that turn it into send
//             offsets, and every assignment's stable place in the expert-sorted order
//             (the GPU-resident metadata);
//   tables    every receiver's counts and offsets, formed from all senders' send
//             offsets by the first kernel that runs after planning (the metadata
//             exchange between ranks, with no host involved);
//   pack      token rows copied into expert-sorted send segments (staged path) or
//             straight into the receiving ranks' buffers (direct path);
//   exchange  staged path: segments copied into the receiving ranks' buffers at
//             device-computed offsets (the all-to-allv), and reversed for the return;
//   combine   gate-weighted sum of each token's k expert rows, float32 accumulate,
//             reading the return buffer (staged) or the expert outputs in place (direct).
// Everything but planning is a row copy or gather bound by HBM bandwidth: rows move as
// 16-byte vectors, one 64-lane wavefront per row (or per piece of a row), with all of a
// row's loads issued before its stores, stores non-temporal (but for the top-k pack's
// scattered stores at streaming sizes), loads non-temporal for buffers too large to stay
// in cache.  Nothing here is a dense contraction, so no matrix-core instruction is used.
// Small steps (decode sizes) are bound by launches and dependent table reads instead of
// bytes; there plan, tables and pack run as one launch in which every block works from
// the routing ids (dispatch_small_kernel).
#include "a2av_internal.h"

#include <algorithm>

namespace a2av {
namespace {

constexpr int kWave = 64;
constexpr int kRowsPerBlock = 4;     // 256-thread blocks, one wavefront per row (measured: with
                                     // a row's loads all in flight, 256-thread blocks move
                                     // streaming rows 4-5 % faster than 1024-thread ones)
constexpr int kBlock = kWave * kRowsPerBlock;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int B> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };

// How rows are cut into chunks, one wavefront per chunk: when a kernel has too few rows
// to give every CU several wavefronts (decode sizes), each row is split into cpr chunks
// of cv vectors (a multiple of 64, so every lane moves the same count); otherwise cpr = 1.
struct Split {
    int nvec;   // vectors per row
    int cpr;    // chunks per row
    int cv;     // vectors per chunk
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// ---- debug build ---------------------------------------------------------------------
// Built with -DA2AV_DEBUG=1 (liba2av_debug.so), the kernels of the path check every row
// index they form against the rows of the buffer it addresses before the access, and
// every table value they turn into an index against its range; a failed check ORs
// kStBounds into the call's status word and the access is skipped.  The release build
// compiles the checks away: there the same indices are in range by construction
// (receive places checked against the capacity, send places against the rows a sender
// sends, ids against [0, E)).
#ifndef A2AV_DEBUG
#define A2AV_DEBUG 0
#endif
// Whether 0 <= i < n (always true in the release build).
__device__ __forceinline__ bool row_ok(uint32_t* status, int64_t i, int64_t n) {
    if constexpr (A2AV_DEBUG != 0) {
        if ((uint64_t)i < (uint64_t)n) return true;
        atomicOr(status, kStBounds);
        return false;
    } else {
        return true;
    }
}
// Flags a value that the release code already steps around but that no correct table
// holds (debug build only).
__device__ __forceinline__ void flag_if(uint32_t* status, bool bad) {
    if constexpr (A2AV_DEBUG != 0) {
        if (bad) atomicOr(status, kStBounds);
    }
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

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, const V& v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
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

// ---- the metadata exchange ------------------------------------------------------------
// Rows rank d gets from sender s: the length of s's segment for d.
__device__ __forceinline__ int seg_len(const int32_t* send_off, int R, int s, int d) {
    const int32_t* so = send_off + (int64_t)s * (R + 1);
    return so[d + 1] - so[d];
}

// recv_off[d][s] computed from the senders' send offsets (whole wavefront, uniform
// result): the rows d receives from the senders before s.
// Index searches read their table entries unconditionally, at an index clamped into the
// table, and mask the result: a read guarded by a lane condition compiles to a branch
// with a wait of its own.
__device__ __forceinline__ int64_t recv_base(const int32_t* send_off, int R, int d, int s, int lane) {
    int acc = 0;
    for (int c0 = 0; c0 < s; c0 += kWave) {
        const int sp = c0 + lane;
        const int c = seg_len(send_off, R, min(sp, s - 1), d);
        acc += sp < s ? c : 0;
    }
    return wave_sum(acc);
}

// Receiver d's table row (one wavefront): recv_counts[d][s], recv_off[d][s] (exclusive
// prefix over s) and the total; flags a receiver whose rows exceed its capacity.
__device__ void write_recv_tables(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status, int d,
                                  int lane) {
    const int R = sh.R;
    int carry = 0;
    for (int s0 = 0; s0 < R; s0 += kWave) {
        const int s = s0 + lane;
        const int c = s < R ? seg_len(tb.send_off, R, s, d) : 0;
        const int incl = wave_inclusive_scan(c);
        if (s < R) {
            const int off = carry + incl - c;
            tb.recv_counts[(int64_t)d * R + s] = c;
            tb.recv_off[(int64_t)d * (R + 1) + s] = off;
            if (out.recv_counts) out.recv_counts[(int64_t)d * R + s] = c;
            if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + s] = off;
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
        tb.recv_off[(int64_t)d * (R + 1) + R] = carry;
        if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + R] = carry;
        if ((int64_t)carry > sh.cap) atomicOr(status, 2u);
    }
}

// Blocks that build the receive tables, one wavefront per receiver, in the grid of the
// kernel that follows planning: after the row blocks in pack (so that pack's row blocks
// keep the same block numbers as those of the kernels reading its rows), first in the
// bare collective.
__host__ __device__ __forceinline__ int64_t table_blocks(int R) { return (R + kRowsPerBlock - 1) / kRowsPerBlock; }

// ------------------------------------------------------------------------------------
// plan: histogram, scans, stable positions and send offsets of every rank.
//
// Positions are a stable counting sort by (expert, token, slot).  A rank's assignments
// are cut into C chunks, one block each (C = 1 for a short rank).  Each wavefront of a
// block owns a contiguous run of its chunk and takes it in batches of S x 64, loading a
// whole batch before using it.  Lanes holding the same expert find each other with one
// ballot per bit of the expert id (the AND of the matching ballots is the set of lanes
// with an equal id); a lane's rank among them is the popcount of that set below it.  The
// lowest such lane adds the group size to the wavefront's private LDS counter for that
// expert, so no atomics decide a place and the result does not depend on timing.
// Counters of all wavefronts are then scanned in (expert, wavefront) order into final
// bases.  With C > 1 every block also counts the whole rank's histogram, and the part
// of it in the chunks before its own, by LDS atomic increments (counts do not depend on
// order): the rank's expert starts and its chunk's bases follow without waiting for any
// other block.  (Measured at 8192 assignments per rank: one block per rank spends ~6 us
// in the ballot matching alone, 16 wavefronts sharing one CU.)
// ------------------------------------------------------------------------------------
struct PlanArgs {
    Shape sh;
    Tables tb;
    Outputs out;
    const int32_t* ids;
    uint32_t* status;
    bool inverse;   // also write inv (and dest = -1 for dropped slots) for the gather pack
};

// Planning of chunk c (of C) of rank s by the whole block; lds holds (waves + 1) * E
// ints, (waves + 2) * E when C > 1; wsum 17.  Block c == 0 writes the rank's tables.
template <int S>
__device__ void plan_rank(const PlanArgs& a, int s, int c, int C, int* lds, int* wsum) {
    const Shape& sh = a.sh;
    const int E = sh.E, R = sh.R;
    const int tid = threadIdx.x, nt = blockDim.x, lane = lane_id(), w = tid / kWave, nw = nt / kWave;
    int* cw = lds;               // [nw][E] per-wavefront counters, later bases
    int* tot = lds + nw * E;     // [E] per-expert totals of the rank, later exclusive offsets
    int* bef = tot + E;          // [E] (C > 1) the rank's rows per expert in the chunks before c

    for (int i = tid; i < (nw + (C > 1 ? 2 : 1)) * E; i += nt) lds[i] = 0;
    __syncthreads();

    const int64_t TK = sh.TK;
    const int32_t* ids = a.ids + (int64_t)s * TK;
    int32_t* pos = a.tb.pos + (int64_t)s * TK;
    const int64_t clen = ((TK + C - 1) / C + kWave - 1) / kWave * kWave;
    const int64_t c0 = min(TK, (int64_t)c * clen), c1 = min(TK, c0 + clen);
    if (C > 1) {
        // the whole rank's histogram and that of the chunks before c; ids are read in
        // rounds of kU per thread, all issued before any is used, at clamped indices
        constexpr int kU = 8;
        for (int64_t i0 = 0; i0 < TK; i0 += (int64_t)nt * kU) {
            int ev[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) ev[u] = ids[min(i0 + (int64_t)u * nt + tid, TK - 1)];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t i = i0 + (int64_t)u * nt + tid;
                if (i < TK && (unsigned)ev[u] < (unsigned)E) {
                    atomicAdd(&tot[ev[u]], 1);
                    if (i < c0) atomicAdd(&bef[ev[u]], 1);
                }
            }
        }
    }
    const int64_t chunk = ((c1 - c0 + nw - 1) / nw + kWave - 1) / kWave * kWave;
    const int64_t a0 = min(c1, c0 + (int64_t)w * chunk), a1 = min(c1, a0 + chunk);
    const int64_t batch = (int64_t)S * kWave;
    const bool one_batch = a1 - a0 <= batch;
    int* mine = cw + w * E;
    bool bad = false;
    int ev[S], rk[S];

    // pass 1: rank of every assignment among equal experts inside its wavefront's run
    for (int64_t b0 = a0; b0 < a1; b0 += batch) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int64_t i = b0 + u * kWave + lane;
            ev[u] = i < a1 ? ids[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int64_t i = b0 + u * kWave + lane;
            const bool valid = i < a1;
            const int e = ev[u];
            const bool in = valid && e >= 0 && e < E;
            bad |= valid && !in;
            uint64_t match = __ballot(in);
            for (int b = 0; b < sh.nbits; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t m = __ballot(in && bit);
                match &= bit ? m : ~m;
            }
            rk[u] = -1;
            if (in) {
                const int r = __popcll(match & lanes_below(lane));
                const int cnt = mine[e];
                rk[u] = cnt + r;
                if (r == 0) mine[e] = cnt + __popcll(match);
            }
            if (!one_batch && valid) pos[i] = rk[u];
        }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(a.status, 1u);
    __syncthreads();

    // per expert: wavefront bases (exclusive over wavefronts); with one chunk, the
    // rank's count is their sum
    for (int e = tid; e < E; e += nt) {
        int run = 0;
        for (int v = 0; v < nw; ++v) { const int cc = cw[v * E + e]; cw[v * E + e] = run; run += cc; }
        if (C == 1) tot[e] = run;
    }
    __syncthreads();
    if (c == 0) {
        for (int e = tid; e < E; e += nt) {
            a.tb.cnt[(int64_t)s * E + e] = tot[e];
            if (a.out.split) a.out.split[(int64_t)s * E + e] = tot[e];
        }
    }
    const int total = block_exclusive_scan(tot, E, wsum);   // tot[e] = first row of expert e

    // send segments: destination d holds experts d*epr .. d*epr+epr-1, which are
    // consecutive in the sorted order
    if (c == 0) {
        for (int d = tid; d <= R; d += nt) a.tb.send_off[(int64_t)s * (R + 1) + d] = d < R ? tot[d * sh.epr] : total;
        for (int e = tid; e <= E; e += nt) a.tb.eoff[(int64_t)s * (E + 1) + e] = e < E ? tot[e] : total;
    }
    for (int i = tid; i < nw * E; i += nt) cw[i] += tot[i % E] + (C > 1 ? bef[i % E] : 0);
    __syncthreads();

    // pass 2: final positions; for the gather pack also the inverse (which assignment
    // sits at each send place) and, since no send place leads to a dropped slot, its
    // empty receive row
    int32_t* inv = a.tb.inv + (int64_t)s * TK;
    int64_t* dest = a.tb.dest + (int64_t)s * TK;
    auto put = [&](int64_t i, int p) {
        pos[i] = p;
        if (a.inverse) {
            if (p >= 0) {
                if (row_ok(a.status, p, TK)) inv[p] = (int32_t)i;
            } else {
                dest[i] = -1;
            }
        }
    };
    if (one_batch) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int64_t i = a0 + u * kWave + lane;
            if (i < a1) put(i, rk[u] >= 0 ? mine[ev[u]] + rk[u] : -1);
        }
    } else {
        for (int64_t i = a0 + lane; i < a1; i += kWave) {
            const int e = ids[i];
            put(i, (e >= 0 && e < E) ? mine[e] + pos[i] : -1);
        }
    }
}

// One block per (rank, chunk): block b plans chunk b % C of rank b / C.
template <int S>
__global__ void __launch_bounds__(1024) plan_kernel(PlanArgs a, int C) {
    extern __shared__ int lds[];
    __shared__ int wsum[17];
    plan_rank<S>(a, blockIdx.x / C, blockIdx.x % C, C, lds, wsum);
}

// Expert-major receive places.  Receiver d's rows are grouped by local expert, then by
// sender, then in the sender's order, so the place of the first row sender s sends to
// expert e is the sum of cnt[s'][e'] over the (local expert, sender) pairs before (e, s)
// in that order: an exclusive scan over d's epr x R pairs.  One wavefront per receiver;
// lane l takes pair c0 + l of each run of 64, the run's counts are loaded together (the
// next run's while this one is scanned), and a wavefront scan with a carry between runs
// gives xbase[s][e] and, at each expert's first sender, recv_eoff[d][le].  Run by the
// receiver-table wavefronts of pack, so the tables are there for every later kernel.
__device__ void write_expert_major_tables(const Shape& sh, const Tables& tb, int d, int lane) {
    const int R = sh.R, E = sh.E, epr = sh.epr;
    const int pairs = epr * R;   // = E
    auto load = [&](int i) -> int {
        if (i >= pairs) return 0;
        const int le = i / R, s = i - le * R;
        return tb.cnt[(int64_t)s * E + d * epr + le];
    };
    int carry = 0;
    int c = load(lane);
    for (int c0 = 0; c0 < pairs; c0 += kWave) {
        const int next = load(c0 + kWave + lane);
        const int i = c0 + lane;
        const int incl = wave_inclusive_scan(c);
        if (i < pairs) {
            const int le = i / R, s = i - le * R;
            const int start = carry + incl - c;
            tb.xbase[(int64_t)s * E + d * epr + le] = start;
            if (s == 0) tb.recv_eoff[(int64_t)d * (epr + 1) + le] = start;
        }
        carry += __shfl(incl, kWave - 1, kWave);
        c = next;
    }
    if (lane == 0) tb.recv_eoff[(int64_t)d * (epr + 1) + epr] = carry;
}

// The expert of send row p of sender s, given its destination d: the number of d's
// experts whose block in the sender's order ends at or before p (one ballot per 64).
__device__ __forceinline__ int expert_of(const Shape& sh, const Tables& tb, int64_t s, int64_t p, int d, int lane) {
    const int32_t* eo = tb.eoff + s * (sh.E + 1) + (int64_t)d * sh.epr;
    int le = 0;
    for (int c0 = 0; c0 < sh.epr; c0 += kWave) {
        const int i = c0 + lane;
        const int64_t end = eo[min(i, sh.epr - 1) + 1];
        le += __popcll(__ballot((i < sh.epr) & (end <= p)));
    }
    return d * sh.epr + le;
}

// Expert-major receive place of send row p (destination d) of sender s.
__device__ __forceinline__ int64_t expert_major_place(const Shape& sh, const Tables& tb, int64_t s, int64_t p, int d,
                                                      int lane) {
    const int e = expert_of(sh, tb, s, p, d, lane);
    return (int64_t)tb.xbase[s * sh.E + e] + (p - tb.eoff[s * (sh.E + 1) + e]);
}

// The same place computed from the plan's counts alone (for the kernel that runs
// beside the table writers): d's rows for its experts below e over all senders, plus
// e's rows from the senders before s, plus p's rank in s's run of e; the first two are
// summed over d's (local expert, sender) pairs, one pair per lane at a time.
__device__ __forceinline__ int64_t expert_major_place_counted(const Shape& sh, const Tables& tb, int64_t s,
                                                              int64_t p, int d, int lane) {
    const int e = expert_of(sh, tb, s, p, d, lane);
    const int R = sh.R, E = sh.E, epr = sh.epr, le = e - d * epr;
    // pair i = l2 * R + s2 comes before (le, s) exactly when i < le * R + s
    const int lim = le * R + (int)s;
    int acc = 0;
    for (int c0 = 0; c0 < lim; c0 += kWave) {
        const int i = min(c0 + lane, lim - 1);
        const int l2 = i / R, s2 = i - l2 * R;
        const int c = tb.cnt[(int64_t)s2 * E + d * epr + l2];
        acc += c0 + lane < lim ? c : 0;
    }
    return (int64_t)wave_sum(acc) + (p - tb.eoff[s * (E + 1) + e]);
}

// The bare collective's planning: send offsets from caller counts, one block per sender.
struct CountsArgs {
    Shape sh;
    Tables tb;
    const int32_t* send_counts;
    uint32_t* status;
};

__global__ void __launch_bounds__(kBlock) plan_from_counts_kernel(CountsArgs a) {
    __shared__ int sc[kMaxRanks + 1];
    __shared__ int wsum[5];
    __shared__ int64_t part[kBlock / kWave];
    const int R = a.sh.R, tid = threadIdx.x, s = blockIdx.x, lane = lane_id(), w = tid / kWave;
    // counts must be non-negative and fit the sender's rows: each thread checks and sums
    // its share in 64 bits, then the block combines the shares
    int64_t sum = 0;
    int neg = 0;
    for (int d = tid; d < R; d += kBlock) {
        const int c = a.send_counts[(int64_t)s * R + d];
        sc[d] = c;
        neg |= c < 0;
        sum += c;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane == 0) part[w] = sum;
    const bool any_neg = __syncthreads_or(neg) != 0;   // also the barrier for part[] and sc[]
    int64_t total_rows = 0;
#pragma unroll
    for (int i = 0; i < kBlock / kWave; ++i) total_rows += part[i];
    const bool good = !any_neg && total_rows <= a.sh.TK;
    if (!good) {
        if (tid == 0) atomicOr(a.status, 1u);
        for (int d = tid; d < R; d += kBlock) sc[d] = 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(sc, R, wsum);
    for (int d = tid; d <= R; d += kBlock) a.tb.send_off[(int64_t)s * (R + 1) + d] = d < R ? sc[d] : total;
}

// ------------------------------------------------------------------------------------
// Row movement.  One wavefront per row; lane l moves vectors l, l+64, ...; U vectors
// per lane are loaded before any is stored.
// ------------------------------------------------------------------------------------
// Load U vectors of a chunk starting at `base` (lane l: vectors base + l, base + 64 + l,
// ...; only those below v1 are used), every load issued unconditionally at an index
// clamped below v1 so that all U are in flight together: a load under a lane condition
// compiles to a branch that first waits for every earlier load.  (Measured on 10 KiB
// prefill rows with 256-thread blocks: pack 244 -> 240 us, exchange 240 -> 229 us, return
// 229 -> 219 us.  The combine keeps its guarded loads: there, all in flight was slower.)
template <int U, bool NT, typename V>
__device__ __forceinline__ void load_chunk(V (&r)[U], const V* __restrict__ src, int base, int v1, int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = ld<NT>(src + min(base + u * kWave + lane, v1 - 1));
}

// Copy vectors [v0, v1) of a row.
template <typename V, int U, bool NT>
__device__ __forceinline__ void copy_row(V* __restrict__ dst, const V* __restrict__ src, int v0, int v1, int lane) {
    for (int base = v0; base < v1; base += kWave * U) {
        V r[U];
        load_chunk<U, NT>(r, src, base, v1, lane);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < v1) st<true>(dst + v, r[u]);
        }
    }
}

template <typename V>
__device__ __forceinline__ void zero_row(V* __restrict__ dst, int v0, int v1, int lane) {
    for (int v = v0 + lane; v < v1; v += kWave) dst[v] = V{};
}

// The wavefront's (row, chunk) and its vector range.
struct Piece {
    int64_t row;
    int v0, v1;
};
__device__ __forceinline__ Piece piece_of(int64_t wave, const Split& sp) {
    Piece p;
    p.row = wave / sp.cpr;
    const int c = (int)(wave - p.row * sp.cpr);
    p.v0 = c * sp.cv;
    p.v1 = min(sp.nvec, p.v0 + sp.cv);
    return p;
}

// Which destination segment holds send row p of a sender: the number of segment ends
// send_off[d+1] at or below p (one ballot per 64 destinations).
__device__ __forceinline__ int segment_of(const int32_t* so, int R, int64_t p, int lane) {
    int d = 0;
    for (int c0 = 0; c0 < R; c0 += kWave) {
        const int i = c0 + lane;
        const int64_t end = so[min(i, R - 1) + 1];
        d += __popcll(__ballot((i < R) & (end <= p)));
    }
    return d;
}

// pack: row x[s][t] to its k places: the sender's send buffer (staged) or the
// receivers' buffers (direct).  The blocks after the row blocks build the receive tables.
// NTS: non-temporal row stores (see launch_pack for when they are not).
template <typename V, int U, bool NT, bool NTS, bool DIRECT, int RPB>
__global__ void __launch_bounds__(RPB * kWave) pack_kernel(const V* __restrict__ x, V* __restrict__ dst, Shape sh,
                                                           Tables tb, Outputs out, uint32_t* status, Split sp) {
    const int lane = lane_id();
    const int64_t rblk = ((int64_t)sh.R * sh.T * sp.cpr + RPB - 1) / RPB;
    if ((int64_t)blockIdx.x >= rblk) {
        const int64_t d = ((int64_t)blockIdx.x - rblk) * RPB + threadIdx.x / kWave;
        if (d < sh.R) {
            write_recv_tables(sh, tb, out, status, (int)d, lane);
            if (sh.layout) write_expert_major_tables(sh, tb, (int)d, lane);
        }
        return;
    }
    const Piece pc = piece_of((int64_t)blockIdx.x * RPB + threadIdx.x / kWave, sp);
    const int64_t n = pc.row;
    if (n >= (int64_t)sh.R * sh.T) return;
    const int64_t s = n / sh.T;
    const int k = sh.k;
    const int R = sh.R;
    const int nvec = sp.nvec;
    const int my = lane < k ? tb.pos[n * k + lane] : -1;
    const V* src = x + n * nvec;
    const int32_t* so = tb.send_off + s * (R + 1);
    for (int base = pc.v0; base < pc.v1; base += kWave * U) {
        // the first piece of a row records where its slots went (for the combine)
        const bool record = base == 0 && lane == 0;
        V r[U];
        load_chunk<U, NT>(r, src, base, pc.v1, lane);
        for (int j = 0; j < k; ++j) {
            const int pj = __builtin_amdgcn_readlane(my, j);
            if (pj < 0 || pj >= sh.TK) {              // dropped slot (never out of the buffer)
                flag_if(status, pj >= sh.TK);
                if (DIRECT && record) tb.dest[n * k + j] = -1;
                continue;
            }
            V* row;
            if constexpr (DIRECT) {
                const int d = segment_of(so, R, pj, lane);
                const int64_t q = d >= R ? -1          // not a sent row (tables always place it)
                                         : sh.layout ? expert_major_place_counted(sh, tb, s, pj, d, lane)
                                                     : recv_base(tb.send_off, R, d, (int)s, lane) + (pj - so[d]);
                flag_if(status, q < 0);
                const int64_t rr = q >= 0 && q < sh.cap ? (int64_t)d * sh.cap + q : -1;   // past capacity: flagged
                if (record) tb.dest[n * k + j] = rr;
                if (rr < 0 || !row_ok(status, rr, (int64_t)R * sh.cap)) continue;
                row = dst + rr * nvec;
            } else {
                row = dst + (s * sh.TK + pj) * nvec;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * kWave + lane;
                if (v < pc.v1) st<NTS>(row + v, r[u]);
            }
        }
    }
}

// pack, gather form (top-1, where the pack is a permutation of the rows): one wavefront
// per send place p of sender s, reading the token the planner placed there, so that
// stores go out in place order and only the loads are scattered over the experts' runs
// (the access shape of the return exchange).  Places past the rows s sends hold nothing
// and are skipped; the receive tables are built by the blocks after the rows, as in pack.
template <typename V, int U, bool NT, bool DIRECT, int RPB>
__global__ void __launch_bounds__(RPB * kWave) pack_gather_kernel(const V* __restrict__ x, V* __restrict__ dst,
                                                                  Shape sh, Tables tb, Outputs out, uint32_t* status,
                                                                  Split sp) {
    const int lane = lane_id();
    const int64_t rows = (int64_t)sh.R * sh.TK;
    const int64_t rblk = (rows * sp.cpr + RPB - 1) / RPB;
    if ((int64_t)blockIdx.x >= rblk) {
        const int64_t d = ((int64_t)blockIdx.x - rblk) * RPB + threadIdx.x / kWave;
        if (d < sh.R) {
            write_recv_tables(sh, tb, out, status, (int)d, lane);
            if (sh.layout) write_expert_major_tables(sh, tb, (int)d, lane);
        }
        return;
    }
    const Piece pc = piece_of((int64_t)blockIdx.x * RPB + threadIdx.x / kWave, sp);
    const int64_t g = pc.row;
    if (g >= rows) return;
    const int R = sh.R;
    const int nvec = sp.nvec;
    const int64_t s = g / sh.TK, p = g - s * sh.TK;
    const int32_t* so = tb.send_off + s * (R + 1);
    if (p >= so[R]) return;                          // not a sent row
    const int32_t t = tb.inv[g];
    if (!row_ok(status, t, sh.T)) return;
    const int64_t n = s * sh.T + t;                  // its token (k = 1: the assignment is the token)
    int64_t row = g;
    if constexpr (DIRECT) {
        const int d = segment_of(so, R, p, lane);    // < R, since p < so[R]
        const int64_t q = sh.layout ? expert_major_place_counted(sh, tb, s, p, d, lane)
                                    : recv_base(tb.send_off, R, d, (int)s, lane) + (p - so[d]);
        flag_if(status, q < 0);
        row = q >= 0 && q < sh.cap ? (int64_t)d * sh.cap + q : -1;   // past capacity: flagged by the tables
        if (pc.v0 == 0 && lane == 0) tb.dest[n] = row;
        if (row < 0 || !row_ok(status, row, (int64_t)R * sh.cap)) return;
    }
    copy_row<V, U, NT>(dst + row * nvec, x + n * nvec, pc.v0, pc.v1, lane);
}

// ---- one-launch dispatch for small steps -------------------------------------------
// At decode sizes the step is short enough that every dependent read of a table just
// written by another kernel shows: such a table sits in another XCD's L2 or in HBM,
// and the read costs microseconds.  So a small step's dispatch is one launch in which
// no block reads what another block of the launch writes; every block works from the
// routing ids directly:
//   blocks [0, R)          planning of one rank each (the tables later kernels use);
//   next R                 one receiver's tables each, counted from the ids;
//   from `lead` on         rows: each wavefront finds where its token's k assignments
//                          go by counting the assignments that come before them in the
//                          destination's order (the block's four wavefronts split the
//                          count when they hold pieces of one row), and copies the row.
// `lead` is a multiple of 8, so a row keeps the block number (and with it the XCD) it
// has in the combine.  Row stores are non-temporal, as everywhere.

// The step's ids, copied into LDS by the whole block (one round of loads).
__device__ __forceinline__ void stage_ids(const int32_t* __restrict__ ids, int64_t A, int* sids) {
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < A; i += blockDim.x) sids[i] = ids[i];
}

// Places of NS assignments of one token row of sender s in their destinations' order,
// counted over the ids (in LDS) by the whole wavefront in one pass, one ballot per slot
// per 64 ids (the counts are wavefront-uniform).  Assignment j has index me0 + j, expert
// e[j] (< 0: none) and destination d[j].  Staged: its place in the sender's (expert,
// token, slot) order.  Direct, source-major: rows d gets from the senders before s, then
// s's rows for d's experts below e, then s's earlier rows for e.  Direct, expert-major:
// d's rows for its experts below e, then the earlier rows for e over all senders in
// (sender, token, slot) order.
// `part` of `parts` equal slices of the scanned ids is counted (the caller adds the
// parts up).
template <bool DIRECT, int NS>
__device__ __forceinline__ void count_places(const Shape& sh, const int* sids, int s, int me0, const int* e,
                                             const int* d, int* q, int lane, int part, int parts) {
    const int A = sh.R * (int)sh.TK, TK = (int)sh.TK;
    int lo, hi, before;       // ids scanned, and the index below which every row of d counts
    if (!DIRECT) { lo = s * TK; hi = lo + TK; before = lo; }
    else if (sh.layout) { lo = 0; hi = A; before = 0; }
    else { lo = 0; hi = (s + 1) * TK; before = s * TK; }
    const int slice = (hi - lo + parts - 1) / parts;
    lo += part * slice;
    hi = min(hi, lo + slice);
    // Branch-free test (short-circuit conditions compile to an exec-mask branch per id run
    // and slot, which made the count the slowest part of the launch): id i counts for
    // slot j when it is scanned, names one of the slot's candidate experts (one unsigned
    // range compare), and either belongs to a whole earlier sender or precedes the slot
    // in (expert, index) order.  That order is one unsigned key, expert << 16 | index -
    // before: the offset is below 2^16 (at most 4096 assignments) and only ids inside the
    // expert range, all below 2^15, have their key compared.
    unsigned elo[NS], span[NS], kme[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const bool some = e[j] >= 0;
        elo[j] = some && DIRECT ? (unsigned)(d[j] * sh.epr) : 0u;
        span[j] = some ? (unsigned)(DIRECT ? sh.epr : sh.E) : 0u;   // 0: counts nothing
        kme[j] = ((unsigned)e[j] << 16) | (unsigned)(me0 + j - before);
        q[j] = 0;
    }
    constexpr int kRuns = 4;   // 64-id runs read before any is used
    for (int i0 = lo; i0 < hi; i0 += kRuns * kWave) {
        int v[kRuns];
#pragma unroll
        for (int u = 0; u < kRuns; ++u) {
            const int i = i0 + u * kWave + lane;
            v[u] = sids[i < hi ? i : lo];
        }
#pragma unroll
        for (int u = 0; u < kRuns; ++u) {
            const int i = i0 + u * kWave + lane;
            const bool live = i < hi, early = i < before;
            const unsigned key = ((unsigned)v[u] << 16) | (unsigned)(i - before);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const bool hit = live & ((unsigned)v[u] - elo[j] < span[j]) & (early | (key < kme[j]));
                q[j] += __popcll(__ballot(hit));
            }
        }
    }
}

// Receiver d's tables counted from the ids (in LDS) by the whole block into `hist`
// (epr x R ints of LDS, zeroed by the caller): hist[le * R + s] = rows sender s sends to
// d's local expert le, by LDS atomic increments (independent of one another, so they
// pipeline; a loop that waits on LDS every step is slow here, where the row
// wavefronts keep the LDS busy).  Each thread takes every blockDim.x-th id (measured at
// 64 receivers x 2048 ids: one wavefront per receiver left the table blocks ~0.8 us
// behind the rows).  count_tables_write then forms recv_counts / recv_off as
// write_recv_tables does and, for expert-major buffers, xbase and recv_eoff as
// write_expert_major_tables does; the caller puts a block barrier between the two.
__device__ __forceinline__ void count_tables_fill(const Shape& sh, const int* sids, int d, int* hist) {
    const int A = sh.R * (int)sh.TK, TK = (int)sh.TK;
    const int elo = d * sh.epr;
    for (int i = threadIdx.x; i < A; i += blockDim.x) {
        const unsigned le = (unsigned)sids[i] - (unsigned)elo;   // any int32 id: no signed overflow
        if (le < (unsigned)sh.epr) atomicAdd(&hist[(int)le * sh.R + i / TK], 1);
    }
}

__device__ void count_tables_write(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status, int d,
                                   int lane, const int* hist) {
    const int R = sh.R, E = sh.E, epr = sh.epr;
    int carry = 0;
    for (int s0 = 0; s0 < R; s0 += kWave) {
        const int s = s0 + lane;
        int c = 0;
        if (s < R)
            for (int le = 0; le < epr; ++le) c += hist[le * R + s];
        const int incl = wave_inclusive_scan(c);
        if (s < R) {
            const int off = carry + incl - c;
            tb.recv_counts[(int64_t)d * R + s] = c;
            tb.recv_off[(int64_t)d * (R + 1) + s] = off;
            if (out.recv_counts) out.recv_counts[(int64_t)d * R + s] = c;
            if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + s] = off;
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
        tb.recv_off[(int64_t)d * (R + 1) + R] = carry;
        if (out.recv_off) out.recv_off[(int64_t)d * (R + 1) + R] = carry;
        if ((int64_t)carry > sh.cap) atomicOr(status, 2u);
    }
    if (!sh.layout) return;
    // expert-major: exclusive scan over (local expert, sender) pairs, expert-major
    const int pairs = epr * R;
    carry = 0;
    for (int c0 = 0; c0 < pairs; c0 += kWave) {
        const int i = c0 + lane;
        const int c = i < pairs ? hist[i] : 0;
        const int incl = wave_inclusive_scan(c);
        if (i < pairs) {
            const int le = i / R, s = i - le * R;
            const int start = carry + incl - c;
            tb.xbase[(int64_t)s * E + d * epr + le] = start;
            if (s == 0) tb.recv_eoff[(int64_t)d * (epr + 1) + le] = start;
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) tb.recv_eoff[(int64_t)d * (epr + 1) + epr] = carry;
}

// LDS (ints) of the one-launch dispatch: planning needs 5 rows of E counters, a table
// block one histogram of E plus the ids, a row block the ids and its wavefronts' partial
// counts (4 x 64).
__host__ __device__ __forceinline__ int64_t small_lds_ints(int64_t E, int64_t A) {
    const int64_t plan = (kRowsPerBlock + 1) * E, tables = E + A;
    const int64_t rows = A + kRowsPerBlock * kMaxTopK;
    const int64_t m = plan > tables ? plan : tables;
    return m > rows ? m : rows;
}

template <typename V, int U, bool DIRECT>
__global__ void __launch_bounds__(kBlock) dispatch_small_kernel(const V* __restrict__ x, V* __restrict__ dst,
                                                                PlanArgs a, Split sp, int lead) {
    extern __shared__ int lds[];
    __shared__ int wsum[17];
    const Shape& sh = a.sh;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int R = sh.R;
    const int64_t A = (int64_t)R * sh.TK;
    if ((int)blockIdx.x < R) {                      // planning of one rank
        plan_rank<1>(a, blockIdx.x, 0, 1, lds, wsum);
        return;
    }
    if ((int)blockIdx.x < lead) {                   // receiver d's tables
        const int d = (int)blockIdx.x - R;
        if (d >= R) return;                         // padding up to `lead` (whole block)
        int* hist = lds;                            // epr x R = E ints
        int* sids = lds + sh.E;
        for (int i = threadIdx.x; i < sh.E; i += blockDim.x) hist[i] = 0;
        stage_ids(a.ids, A, sids);
        __syncthreads();
        count_tables_fill(sh, sids, d, hist);
        __syncthreads();
        if (w == 0) count_tables_write(sh, a.tb, a.out, a.status, d, lane, hist);
        return;
    }
    const Piece pc = piece_of(((int64_t)blockIdx.x - lead) * kRowsPerBlock + w, sp);
    const int64_t n = pc.row;
    const bool live = n < (int64_t)R * sh.T;
    const int64_t s = n / sh.T;
    const int k = sh.k, nvec = sp.nvec;
    // when a row is cut into a multiple of 4 pieces, a block's 4 wavefronts hold pieces
    // of the same row and each counts a quarter of the ids
    const bool coop = sp.cpr % kRowsPerBlock == 0;
    const int part = coop ? w : 0, parts = coop ? kRowsPerBlock : 1;
    int* partial = lds + A;                         // [4][kMaxTopK] per-wavefront counts
    const V* src = x + n * nvec;
    V r[U];
    int base = pc.v0;
    if (live) load_chunk<U, false>(r, src, base, pc.v1, lane);   // live is uniform per wavefront
    stage_ids(a.ids, A, lds);
    __syncthreads();
    if (!live) return;                              // uniform over the block when coop
    // slot j's expert and destination (lane j), and its count (lane 0 of each
    // wavefront records the part it counted)
    const int my_v = lane < k ? lds[n * k + lane] : -1;
    const int my_e = my_v >= 0 && my_v < sh.E ? my_v : -1;   // out of range: dropped (planning flags it)
    const int my_d = my_e >= 0 ? my_e / sh.epr : 0;
    int my_q = 0;
    auto place = [&](auto NSC, int j0) {
        constexpr int NS = decltype(NSC)::value;
        int e[NS], d[NS], q[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            e[j] = __builtin_amdgcn_readlane(my_e, j0 + j);
            d[j] = __builtin_amdgcn_readlane(my_d, j0 + j);
        }
        count_places<DIRECT, NS>(sh, lds, (int)s, (int)(n * k + j0), e, d, q, lane, part, parts);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (coop && lane == 0) partial[w * kMaxTopK + j0 + j] = q[j];
            if (lane == j0 + j) my_q = q[j];
        }
    };
    int j0 = 0;
    for (; j0 + 4 <= k; j0 += 4) place(std::integral_constant<int, 4>{}, j0);
    if (k - j0 >= 2) { place(std::integral_constant<int, 2>{}, j0); j0 += 2; }
    if (k - j0 == 1) place(std::integral_constant<int, 1>{}, j0);
    if (coop) {
        __syncthreads();
        if (lane < k) {
            my_q = 0;
#pragma unroll
            for (int p = 0; p < kRowsPerBlock; ++p) my_q += partial[p * kMaxTopK + lane];
        }
    }
    // lane j: slot j's destination row, -1 if the slot has none
    int64_t my_row = -1;
    if (lane < k && my_e >= 0) {
        if constexpr (DIRECT) my_row = my_q < sh.cap ? (int64_t)my_d * sh.cap + my_q : -1;   // past capacity
        else my_row = s * sh.TK + my_q;
    }
    // the first piece of a row records where its slots went (for the combine)
    if (DIRECT && pc.v0 == 0 && lane < k) a.tb.dest[n * k + lane] = my_row;
    const int64_t dst_rows = DIRECT ? (int64_t)R * sh.cap : A;
    for (;;) {
        for (int j = 0; j < k; ++j) {
            const int64_t rj = __shfl(my_row, j, kWave);
            if (rj < 0 || !row_ok(a.status, rj, dst_rows)) continue;
            V* row = dst + rj * nvec;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * kWave + lane;
                if (v < pc.v1) st<true>(row + v, r[u]);
            }
        }
        base += kWave * U;
        if (base >= pc.v1) break;
        load_chunk<U, false>(r, src, base, pc.v1, lane);
    }
}

// exchange (staged path): send row (s, p) <-> receive row (d, q).  Forward copies send
// -> recv and drops rows past the capacity; reverse copies recv-layout expert outputs
// back to the send places and writes zeros where a row was dropped.  FIRST: this is the
// first kernel after planning (the bare collective), so the first blocks build the
// receive tables and rows find their receive offset from the send offsets.
// The forward copy below streaming sizes issues the first chunk of its send row's loads
// before it reads any table: the send row is known from the wavefront's index (and lies
// in the library's send buffer whether or not the sender fills it), so the row's load
// latency overlaps the dependent table reads (same-box A/B: edge-shape staged dispatch
// 12.4 -> 11.3 us, 12.9 -> 11.7 expert-major; decode expert-major 14.1 -> 13.0, decode
// source-major unchanged; at prefill the exchange was 2 % slower, so streaming sizes
// keep the table reads first).
template <typename V, int U, bool NT, bool REVERSE, bool FIRST, int RPB>
__global__ void __launch_bounds__(RPB * kWave) exchange_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                               Shape sh, Tables tb, Outputs out, uint32_t* status,
                                                               Split sp) {
    const int lane = lane_id();
    int64_t blk = blockIdx.x;
    if constexpr (FIRST) {
        const int64_t tblk = table_blocks(sh.R);
        if (blk < tblk) {
            const int d = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
            if (d < sh.R) write_recv_tables(sh, tb, out, status, d, lane);
            return;
        }
        blk -= tblk;
    }
    const Piece pc = piece_of(blk * RPB + threadIdx.x / kWave, sp);
    const int64_t g = pc.row;
    if (g >= (int64_t)sh.R * sh.TK) return;
    const int R = sh.R;
    const int nvec = sp.nvec;
    const int64_t s = g / sh.TK, p = g - s * sh.TK;
    constexpr bool kLoadsFirst = !NT && !REVERSE && !FIRST;
    V r0[U];
    if constexpr (kLoadsFirst) load_chunk<U, NT>(r0, src + (s * sh.TK + p) * nvec, pc.v0, pc.v1, lane);
    const int32_t* so = tb.send_off + s * (R + 1);
    int d;
    int64_t q;
    if (!NT && !FIRST && !sh.layout && R <= kWave) {
        // below streaming sizes, source-major, at most 64 ranks: the sender's send offsets
        // (lane l: so[l]) and every receiver's receive offset for this sender (lane l:
        // recv_off[l][s]) in one round of loads, then the segment and the place from
        // registers, where the general form reads them in three dependent rounds
        const int32_t so_l = so[min(lane, R - 1)];
        const int32_t so_end = so[R];
        const int32_t ro_l = tb.recv_off[(int64_t)min(lane, R - 1) * (R + 1) + s];
        if (p >= so_end) return;
        const int32_t up = __shfl(so_l, min(lane + 1, kWave - 1), kWave);
        const int32_t seg_end = lane + 1 < R ? up : so_end;          // so[l + 1]
        d = __popcll(__ballot(lane < R && seg_end <= p));            // < R, since p < so[R]
        q = (int64_t)__shfl(ro_l, d, kWave) + (p - __shfl(so_l, d, kWave));
    } else {
        if (p >= so[R]) return;
        d = segment_of(so, R, p, lane);
        if (FIRST) q = recv_base(tb.send_off, R, d, (int)s, lane) + (p - so[d]);   // the bare collective
        else if (sh.layout) q = expert_major_place(sh, tb, s, p, d, lane);
        else q = (int64_t)tb.recv_off[(int64_t)d * (R + 1) + s] + (p - so[d]);
    }
    const int64_t send_row = s * sh.TK + p, recv_row = (int64_t)d * sh.cap + q;
    flag_if(status, q < 0);
    const bool in_cap = q >= 0 && q < sh.cap;
    if (!row_ok(status, send_row, (int64_t)R * sh.TK) || (in_cap && !row_ok(status, recv_row, (int64_t)R * sh.cap)))
        return;
    if (!REVERSE) {
        if (!in_cap) return;
        if constexpr (kLoadsFirst) {
            V* drow = dst + recv_row * nvec;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = pc.v0 + u * kWave + lane;
                if (v < pc.v1) st<true>(drow + v, r0[u]);
            }
            if (pc.v0 + kWave * U < pc.v1)
                copy_row<V, U, NT>(drow, src + send_row * nvec, pc.v0 + kWave * U, pc.v1, lane);
        } else {
            copy_row<V, U, NT>(dst + recv_row * nvec, src + send_row * nvec, pc.v0, pc.v1, lane);
        }
    } else {
        if (!in_cap) { zero_row<V>(dst + send_row * nvec, pc.v0, pc.v1, lane); return; }
        copy_row<V, U, NT>(dst + send_row * nvec, src + recv_row * nvec, pc.v0, pc.v1, lane);
    }
}

// Forward exchange in receive order (source-major buffers): wavefront g takes the g-th
// written receive row, receivers in order and each receiver's rows front to back; its
// sender is the source segment of recv_off[d][.] that holds its place q, and its send
// place is send_off[s][d] + q - recv_off[d][s].  Loads scatter over the senders'
// segments and stores go out in place order, the return exchange's access shape
// (measured: prefill exchange 228.5 -> 224 us, top-8 exchange 1344 -> 1318 us).
template <typename V, int U, bool NT, int RPB>
__global__ void __launch_bounds__(RPB * kWave) exchange_recv_order_kernel(const V* __restrict__ src,
                                                                          V* __restrict__ dst, Shape sh, Tables tb,
                                                                          uint32_t* status, Split sp) {
    const int lane = lane_id();
    const Piece pc = piece_of((int64_t)blockIdx.x * RPB + threadIdx.x / kWave, sp);
    const int64_t g = pc.row;
    if (g >= (int64_t)sh.R * sh.TK) return;
    const int R = sh.R;
    // receiver d and place q of the g-th written row (receiver d holds min(rows, capacity))
    int64_t carry = 0, q = 0;
    int d = -1;
    for (int c0 = 0; c0 < R; c0 += kWave) {
        const int dl = c0 + lane;
        const int64_t got = tb.recv_off[(int64_t)min(dl, R - 1) * (R + 1) + R];
        const int n = dl < R ? (int)(got < sh.cap ? got : sh.cap) : 0;
        const int incl = wave_inclusive_scan(n);
        const uint64_t past = __builtin_amdgcn_ballot_w64(carry + incl > g);
        if (past) {
            const int l = __builtin_ctzll(past);
            d = c0 + l;
            q = g - carry - __shfl(incl - n, l, kWave);
            break;
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (d < 0) return;                               // past the last written row
    const int32_t* ro = tb.recv_off + (int64_t)d * (R + 1);
    const int s = segment_of(ro, R, q, lane);        // < R: q < ro[R]
    const int64_t p = (int64_t)tb.send_off[(int64_t)s * (R + 1) + d] + (q - ro[s]);
    if (!row_ok(status, s, R) || !row_ok(status, p, sh.TK) || !row_ok(status, q, sh.cap)) return;
    copy_row<V, U, NT>(dst + ((int64_t)d * sh.cap + q) * sp.nvec, src + ((int64_t)s * sh.TK + p) * sp.nvec, pc.v0,
                       pc.v1, lane);
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

// combine: y[s][t] = round(sum_j g_j * row_j) with one float32 FMA per slot in slot
// order, starting from 0.  row_j is the returned row at send place pos_j (staged) or
// the expert output in the receiver's buffer (direct).
template <int B, int DT, int U, bool NT, bool DIRECT, bool PAIRS, int RPB>
__global__ void __launch_bounds__(RPB * kWave) combine_kernel(const typename Vec<B>::T* __restrict__ rows,
                                                         const float* __restrict__ gates,
                                                         typename Vec<B>::T* __restrict__ y, Shape sh, Tables tb,
                                                         uint32_t* status, Split sp) {
    using V = typename Vec<B>::T;
    using El = Elems<B, DT>;
    constexpr int NE = El::N;
    const int lane = lane_id();
    const Piece pc = piece_of((int64_t)blockIdx.x * RPB + threadIdx.x / kWave, sp);
    const int64_t n = pc.row;
    if (n >= (int64_t)sh.R * sh.T) return;
    const int64_t s = n / sh.T;
    const int k = sh.k, R = sh.R;
    const int nvec = sp.nvec;
    const int my_p = lane < k ? tb.pos[n * k + lane] : -1;
    const float my_g = lane < k ? gates[n * k + lane] : 0.0f;
    // row index of each slot (held by lane j): a send place (staged) or the receive row
    // dispatch recorded (direct); -1 = the slot adds nothing
    int64_t my_row = -1;
    if constexpr (DIRECT) {
        if (lane < k) {
            const int64_t r = tb.dest[n * k + lane];
            flag_if(status, r < -1 || r >= (int64_t)R * sh.cap);
            if (r >= 0 && r < (int64_t)R * sh.cap) my_row = r;
        }
    } else {
        flag_if(status, lane < k && (my_p < -1 || my_p >= sh.TK));
        if (my_p >= 0 && my_p < sh.TK) my_row = s * sh.TK + my_p;
    }
    V* out = y + n * nvec;
    for (int base = pc.v0; base < pc.v1; base += kWave * U) {
        float acc[U][NE];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[u][e] = 0.0f;
        // PAIRS (k > 1): slots in pairs, each slot's loads issued before the previous
        // slot's multiply-adds so that a wavefront always has rows in flight; the adds
        // stay in slot order
        auto slot_row = [&](int j) -> const V* {   // null: no slot, or a dropped one
            if (j >= k) return nullptr;
            const int64_t rj = __shfl(my_row, j, kWave);
            return rj < 0 ? nullptr : rows + rj * nvec;
        };
        auto load = [&](V* r, const V* row) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * kWave + lane;
                if (v < pc.v1) r[u] = ld<NT>(row + v);
            }
        };
        auto add = [&](const V* r, int j) {
            const float gj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_g), j));
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[u][e] = __builtin_fmaf(gj, El::get(r[u], e), acc[u][e]);
        };
        if constexpr (PAIRS) {
            V ra[U], rb[U];
            const V* pa = slot_row(0);
            if (pa) load(ra, pa);
            for (int j = 0; j < k; j += 2) {
                const V* pb = slot_row(j + 1);
                if (pb) load(rb, pb);
                if (pa) add(ra, j);
                pa = slot_row(j + 2);
                if (pa) load(ra, pa);
                if (pb) add(rb, j + 1);
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const V* p = slot_row(j);
                if (!p) continue;
                V r[U];
                load(r, p);
                add(r, j);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            if (v < pc.v1) st<true>(out + v, El::pack(acc[u]));
        }
    }
}

// The g-th written receive row of an expert-major buffer, taking receivers in order
// and each receiver's rows front to back (so expert group after expert group): receiver
// d holds n_d = min(rows received, capacity) written rows, the row is q = g - (n_0 + ...
// + n_{d-1}) of the first d whose prefix passes g, and its expert is the local expert
// whose group [recv_eoff[d][le], recv_eoff[d][le + 1]) holds q.  False past the last
// written row.  (Whole wavefront; the result is uniform.)
__device__ bool grouped_row(const Shape& sh, const Tables& tb, int64_t g, int lane, int64_t* row, int* e) {
    const int R = sh.R, epr = sh.epr;
    int64_t carry = 0;
    for (int c0 = 0; c0 < R; c0 += kWave) {
        const int d = c0 + lane;
        const int64_t got = tb.recv_off[(int64_t)min(d, R - 1) * (R + 1) + R];
        const int n = d < R ? (int)(got < sh.cap ? got : sh.cap) : 0;
        const int incl = wave_inclusive_scan(n);
        const uint64_t past = __builtin_amdgcn_ballot_w64(carry + incl > g);
        if (past) {
            const int dl = __builtin_ctzll(past);
            const int dd = c0 + dl;
            const int64_t q = g - carry - __shfl(incl - n, dl, kWave);
            const int32_t* eo = tb.recv_eoff + (int64_t)dd * (epr + 1);
            int le = 0;
            for (int l0 = 0; l0 < epr; l0 += kWave) {
                const int l = l0 + lane;
                const int64_t end = eo[min(l, epr - 1) + 1];
                le += __popcll(__builtin_amdgcn_ballot_w64((l < epr) & (end <= q)));
            }
            *row = (int64_t)dd * sh.cap + q;
            *e = dd * epr + le;
            return true;
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    return false;
}

// Harness expert stand-in over every received row: identity, or scale by 1 + e/256
// with one rounding (the float32 product of a bf16 value and 1 + e/256 is exact).
// Expert-major buffers are walked as a grouped expert op walks them: receiver by
// receiver, each local expert's contiguous group in turn, the expert taken from the
// group starts.  Source-major rows are found from the send side as in the exchange; the
// row's expert is the one whose slice of the sender's expert-sorted segment holds it.
template <int B, int DT, int U>
__global__ void __launch_bounds__(kBlock) expert_kernel(const typename Vec<B>::T* __restrict__ in,
                                                        typename Vec<B>::T* out, Shape sh, Tables tb, Split sp,
                                                        int mode) {
    using V = typename Vec<B>::T;
    using El = Elems<B, DT>;
    constexpr int NE = El::N;
    const int lane = lane_id();
    const Piece pc = piece_of((int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave, sp);
    const int64_t g = pc.row;
    if (g >= (int64_t)sh.R * sh.TK) return;
    const int R = sh.R;
    const int nvec = sp.nvec;
    int64_t row;
    int e;
    if (sh.layout) {
        if (!grouped_row(sh, tb, g, lane, &row, &e)) return;
    } else {
        const int64_t s = g / sh.TK, p = g - s * sh.TK;
        const int32_t* so = tb.send_off + s * (R + 1);
        if (p >= so[R]) return;
        const int d = segment_of(so, R, p, lane);
        e = expert_of(sh, tb, s, p, d, lane);
        const int64_t q = (int64_t)tb.recv_off[(int64_t)d * (R + 1) + s] + (p - so[d]);
        if (q < 0 || q >= sh.cap) return;
        row = (int64_t)d * sh.cap + q;
    }
    if (mode == 0) {
        if (in != out) copy_row<V, U, false>(out + row * nvec, in + row * nvec, pc.v0, pc.v1, lane);
        return;
    }
    const float scale = 1.0f + (float)e / 256.0f;
    const V* src = in + row * nvec;
    V* dst = out + row * nvec;
    for (int v = pc.v0 + lane; v < pc.v1; v += kWave) {
        const V r = src[v];
        float f[NE];
#pragma unroll
        for (int c = 0; c < NE; ++c) f[c] = El::get(r, c) * scale;
        dst[v] = El::pack(f);
    }
}

// Reference row copy (measurement harness): the same row movement as the exchange with
// the identity mapping, for the achievable-bandwidth line next to the path's kernels.
template <int U, bool NT, int RPB>
__global__ void __launch_bounds__(RPB * kWave) reference_copy_kernel(const u32x4* __restrict__ src,
                                                                     u32x4* __restrict__ dst, int64_t rows, Split sp) {
    const Piece pc = piece_of((int64_t)blockIdx.x * RPB + threadIdx.x / kWave, sp);
    if (pc.row >= rows) return;
    copy_row<u32x4, U, NT>(dst + pc.row * sp.nvec, src + pc.row * sp.nvec, pc.v0, pc.v1, lane_id());
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

// Row loads are non-temporal once a kernel's rows are far larger than the caches (the
// 256 MiB last-level cache); smaller steps keep them cacheable.  Row stores are
// non-temporal (the one exception is the top-k pack at streaming sizes, launch_pack): no
// kernel reads back what it writes, and a kernel ends only after its XCDs' L2s have
// written back every dirty line, which at decode sizes costs more than the stores
// themselves (measured: non-temporal stores take about 1 us off each decode launch that
// writes 10 MB).
constexpr int64_t kStreamBytes = 256ll << 20;

// At those sizes the path's copy kernels (pack, exchange, return) run at most two
// 256-thread blocks per CU: each block asks for 64 KiB of dynamic LDS that no kernel
// touches, so a CU's 160 KiB holds two.  Their registers alone would allow four; with
// fewer rows in flight per CU, HBM serves their scattered streams faster (same-box A/B
// on 10 KiB rows: pack 231 -> 218 us, return 219 -> 211 us; on 14 KiB top-8 rows:
// exchange 1320 -> 1302 us, return 1357 -> 1318 us; three blocks per CU sat in between).
// The combine, whose loads go one at a time, keeps full occupancy (capped: top-8
// 778 -> 1155 us), and so does the identity reference copy (capped: 6.28 -> 6.17 TB/s).
constexpr unsigned kCopyLds = 64u << 10;
// The zero-copy top-1 pack, which finds each row's receive place before moving it, does
// best at three blocks per CU (same-box A/B, 10 KiB rows: 231-235 us at two, 224 us at
// three, the step 463 -> 460 us).
constexpr unsigned kDirectPackLds = 48u << 10;

template <typename F>
hipError_t with_nt(int64_t bytes, F&& f) {
    if (bytes >= kStreamBytes) return f(std::true_type{});
    return f(std::false_type{});
}

// Wavefronts a row kernel should have to keep every CU busy on short grids.  The
// combine splits finer: its pieces only read, while every piece of a dispatch row
// repeats that row's placement work (measured at 1,024 rows of 10 KiB: 32 per CU takes
// ~0.5 us off the combine and adds ~1.4 us to the one-launch dispatch).
constexpr int kWavesPerCu = 16;
constexpr int kCombineWavesPerCu = 32;

Split make_split(int64_t row_bytes, int vec, int64_t rows, int num_cu, int waves_per_cu = kWavesPerCu,
                 int min_chunks = 1) {
    Split sp;
    sp.nvec = (int)(row_bytes / vec);
    int cpr = 1;
    if (rows > 0) {
        const int64_t target = (int64_t)num_cu * waves_per_cu;
        cpr = (int)std::max<int64_t>((target + rows - 1) / rows, min_chunks);
        cpr = (int)std::min<int64_t>(cpr, std::max(1, sp.nvec / kWave));
        cpr = std::max(1, cpr);
    }
    int cv = (sp.nvec + cpr - 1) / cpr;
    if (cpr > 1) cv = (cv + kWave - 1) / kWave * kWave;
    sp.cv = cv;
    sp.cpr = (sp.nvec + cv - 1) / cv;
    return sp;
}

inline unsigned piece_blocks(int64_t rows, const Split& sp) { return row_blocks(rows * sp.cpr); }

// The exchanges (and the identity reference copy, which moves rows the same way) cut rows
// of more than 12 vectors per lane in two at streaming sizes.  Same-box sweep, staged
// exchange / return in us, whole rows -> two pieces: top-1 rows of 8 KiB 182 / 189 ->
// 220 / 196, 10 KiB 221 / 213 -> 241 / 219, 12 KiB 266 / 267 -> 266 / 263, 14 KiB
// 326 / 327 -> 309 / 313, 16 KiB 385 / 379 -> 363 / 367; top-8 (16 ranks x 1024 tokens)
// the same way from 14 KiB on (return 646 -> 610 us at 14 KiB, 750 -> 721 at 16 KiB).
// The packs keep whole rows (the top-8 pack was slower split).
Split copy_split(int64_t row_bytes, int vec, int64_t rows, int num_cu) {
    Split sp = make_split(row_bytes, vec, rows, num_cu);
    if (sp.cpr == 1 && rows * row_bytes >= kStreamBytes && sp.nvec > 12 * kWave)
        sp = make_split(row_bytes, vec, rows, num_cu, kWavesPerCu, 2);
    return sp;
}

// Vectors per lane kept in flight: the smallest of 1, 2, 4, 8, 16 covering a chunk.
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

int plan_waves(int32_t E, int rows) {
    return std::max(1, std::min(16, (int)(kPlanLdsBytes / (4 * (int64_t)E)) - rows));
}

// Chunks per rank: one per 1024 assignments (one 64-assignment batch per wavefront of a
// 16-wavefront block), at most 16, since every block of a rank counts all its ids.
static int plan_chunks(int64_t TK) { return (int)std::max<int64_t>(1, std::min<int64_t>(16, (TK + 1023) / 1024)); }

hipError_t launch_plan(const Shape& sh, const Tables& tb, const int32_t* ids, const Outputs& out, uint32_t* status,
                       hipStream_t st) {
    const int C = plan_chunks(sh.TK);
    const int64_t clen = ((sh.TK + C - 1) / C + kWave - 1) / kWave * kWave;
    const int rows = C > 1 ? 2 : 1;   // LDS rows of E counters beside the wavefronts'
    // no more wavefronts than there are 64-assignment slices in a chunk: idle ones would
    // only add barrier and scan work
    const int nw = (int)std::max<int64_t>(1, std::min<int64_t>(plan_waves(sh.E, rows), (clen + kWave - 1) / kWave));
    const size_t lds = (size_t)(nw + rows) * sh.E * sizeof(int);
    PlanArgs a{sh, tb, out, ids, status, gather_pack(sh)};
    const int64_t per_wave = (clen + nw - 1) / nw;
    const int64_t slices = (per_wave + kWave - 1) / kWave;
    const dim3 grid((unsigned)(sh.R * C)), block(nw * kWave);
    if (slices <= 1) hipLaunchKernelGGL(plan_kernel<1>, grid, block, lds, st, a, C);
    else if (slices <= 2) hipLaunchKernelGGL(plan_kernel<2>, grid, block, lds, st, a, C);
    else if (slices <= 4) hipLaunchKernelGGL(plan_kernel<4>, grid, block, lds, st, a, C);
    else if (slices <= 8) hipLaunchKernelGGL(plan_kernel<8>, grid, block, lds, st, a, C);
    else hipLaunchKernelGGL(plan_kernel<16>, grid, block, lds, st, a, C);
    return hipGetLastError();
}


hipError_t launch_plan_from_counts(const Shape& sh, const Tables& tb, const int32_t* send_counts, uint32_t* status,
                                   hipStream_t st) {
    CountsArgs a{sh, tb, send_counts, status};
    hipLaunchKernelGGL(plan_from_counts_kernel, dim3(sh.R), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

// The gather form keeps the stores in place order, which pays once the rows stream from
// HBM (prefill 240 -> 233 us staged, 242 -> 231 us direct); below that the scatter form,
// which loads its token row before reading any table and needs no inverse table from
// the planner, is 1-2 % faster (same-box graph A/B at 8 ranks x 768 / 1,024 / 2,048
// tokens of 10 KiB: zero-copy dispatch 26.9 -> 26.4, 33.7 -> 33.1, 57.4 -> 56.5 us).
bool gather_pack(const Shape& sh) { return sh.k == 1 && (int64_t)sh.R * sh.T * sh.row_bytes >= kStreamBytes; }

static hipError_t launch_pack_gather(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status,
                                     const void* x, void* dst, bool direct, int vec, hipStream_t st) {
    const int64_t rows = (int64_t)sh.R * sh.TK;
    const Split sp = make_split(sh.row_bytes, vec, rows, sh.num_cu);
    const int64_t bytes = rows * sh.row_bytes;
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(sp.cv, [&](auto U) {
            return with_nt(bytes, [&](auto NT) {
                constexpr int u = decltype(U)::value;
                constexpr bool nt = decltype(NT)::value;
                constexpr unsigned lds = nt ? kCopyLds : 0u;   // streaming: two blocks per CU
                constexpr int rpb = kRowsPerBlock;
                const unsigned grid = (unsigned)((rows * sp.cpr + rpb - 1) / rpb + (sh.R + rpb - 1) / rpb);
                if (direct)
                    hipLaunchKernelGGL((pack_gather_kernel<V, u, nt, true, rpb>), dim3(grid), dim3(rpb * kWave),
                                       nt ? kDirectPackLds : 0u, st, (const V*)x, (V*)dst, sh, tb, out, status, sp);
                else
                    hipLaunchKernelGGL((pack_gather_kernel<V, u, nt, false, rpb>), dim3(grid), dim3(rpb * kWave), lds,
                                       st, (const V*)x, (V*)dst, sh, tb, out, status, sp);
                return hipGetLastError();
            });
        });
    });
}

// The top-k pack (k > 1) writes every token row to k places scattered over the experts'
// runs.  At streaming sizes it loads and stores through the caches instead of
// non-temporally: the L2s gather the scattered row stores before they go out (same-box
// A/B at the top-8 shape, 16 x 2048 tokens of 14 KiB, receive capacity twice the mean:
// staged pack 868 -> 788 us, direct 885 -> 791 us; cacheable stores alone 801 / 806 us).
// Every other row kernel writes its rows in place order and is 7-10 % slower with
// cacheable stores (prefill pack 218 -> 238 us, exchange 222 -> 235 us), so keeps
// non-temporal ones.  Two blocks per CU, as the other streaming copies.
hipError_t launch_pack(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status, const void* x,
                       void* dst, bool direct, int vec, hipStream_t st) {
    if (gather_pack(sh)) return launch_pack_gather(sh, tb, out, status, x, dst, direct, vec, st);
    const int64_t N = (int64_t)sh.R * sh.T;
    const Split sp = make_split(sh.row_bytes, vec, N, sh.num_cu);
    const int64_t bytes = N * sh.row_bytes;
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(sp.cv, [&](auto U) {
            return with_nt(bytes, [&](auto STREAMING) {
                constexpr int u = decltype(U)::value;
                constexpr bool streaming = decltype(STREAMING)::value;
                constexpr bool nts = !streaming;                      // streaming: cacheable stores
                constexpr unsigned lds = streaming ? kCopyLds : 0u;   // streaming: two blocks per CU
                constexpr int rpb = kRowsPerBlock;
                const unsigned grid = (unsigned)((N * sp.cpr + rpb - 1) / rpb + (sh.R + rpb - 1) / rpb);
                if (direct)
                    hipLaunchKernelGGL((pack_kernel<V, u, false, nts, true, rpb>), dim3(grid), dim3(rpb * kWave), lds,
                                       st, (const V*)x, (V*)dst, sh, tb, out, status, sp);
                else
                    hipLaunchKernelGGL((pack_kernel<V, u, false, nts, false, rpb>), dim3(grid), dim3(rpb * kWave), lds,
                                       st, (const V*)x, (V*)dst, sh, tb, out, status, sp);
                return hipGetLastError();
            });
        });
    });
}

bool small_dispatch(const Shape& sh, bool direct) {
    // The one launch pays off while counting a row's place over the ids costs less than
    // the planning launch it saves.  A row of the staged path counts over its own
    // sender's ids only; a zero-copy row over every id of the senders before it, once per
    // slot, which long rows (more bytes to move behind the count) hide better.  Same-box
    // graph A/B against plan + pack: decode shape (8 ranks, 10 KiB rows) 320 / 512 tokens
    // per rank top-1 zero-copy 15.2 -> 10.4 / 20.3 -> 17.9 us, staged 26.7 -> 22.8 /
    // 37.5 -> 35.1 us; 16 ranks x 256 and 32 x 128 tokens 20.1 -> 17.5 and 19.9 -> 17.6
    // us; top-2 at 200 tokens 13.9 -> 10.8 us; top-8 (14 KiB rows) 16 ranks x 24 / 32
    // tokens 16.4 -> 12.3 / 18.7 -> 15.8 us; past 4096 assignments the zero-copy count lost
    // (768 tokens 27.0 -> 29.5 us), and so it did with 4 KiB rows (64 ranks x 32 tokens
    // top-2 9.95 -> 11.6 us) while the staged form gained there (21.9 -> 18.2 us).  Each
    // planning block ranks its rank's ids in 64-assignment batches per wavefront (up to
    // 1,024 per rank); the ids stay in LDS beside the counters (at most 16 KiB).
    const int64_t A = (int64_t)sh.R * sh.TK;
    if (sh.T == 0 || sh.TK > 1024 || sh.E > 1024) return false;
    return A <= 2048 || (A <= 4096 && (!direct || sh.row_bytes >= 8192));
}

hipError_t launch_dispatch_small(const Shape& sh, const Tables& tb, const int32_t* ids, const Outputs& out,
                                 uint32_t* status, const void* x, void* dst, bool direct, int vec, hipStream_t st) {
    const int64_t N = (int64_t)sh.R * sh.T;
    Split sp = make_split(sh.row_bytes, vec, N, sh.num_cu);
    // A zero-copy row counts its places over every earlier sender's ids, once per slot;
    // only when a row's pieces fill whole blocks do a block's wavefronts split that count.
    // So a zero-copy row cut into a number of pieces that is not a multiple of a block's
    // wavefronts is cut into exactly one block's worth instead (same-box graph A/B, 16
    // ranks x 16 / 8 / 4 tokens of 14 KiB at top-8: 18.2 -> 8.9, 9.9 -> 6.7, 6.6 -> 6.2 us;
    // top-1 decode and edge shapes unchanged).  The staged rows count over their own
    // sender's ids only and keep the finer cut (12.3 against 11.6 us at 4 tokens).
    if (direct && sp.cpr > 1 && sp.cpr % kRowsPerBlock != 0) {
        Split s4;
        s4.nvec = sp.nvec;
        s4.cv = ((sp.nvec + kRowsPerBlock - 1) / kRowsPerBlock + kWave - 1) / kWave * kWave;
        s4.cpr = (s4.nvec + s4.cv - 1) / s4.cv;
        if (s4.cpr == kRowsPerBlock) sp = s4;
    }
    const int lead = (2 * sh.R + 7) / 8 * 8;   // planning and table blocks, padded to a multiple of 8
    const unsigned grid = (unsigned)(lead + piece_blocks(N, sp));
    const size_t lds = (size_t)small_lds_ints(sh.E, (int64_t)sh.R * sh.TK) * sizeof(int);
    const PlanArgs a{sh, tb, out, ids, status, false};   // the rows here place themselves
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(sp.cv, [&](auto U) {
            constexpr int u = decltype(U)::value;
            if (direct)
                hipLaunchKernelGGL((dispatch_small_kernel<V, u, true>), dim3(grid), dim3(kBlock), lds, st,
                                   (const V*)x, (V*)dst, a, sp, lead);
            else
                hipLaunchKernelGGL((dispatch_small_kernel<V, u, false>), dim3(grid), dim3(kBlock), lds, st,
                                   (const V*)x, (V*)dst, a, sp, lead);
            return hipGetLastError();
        });
    });
}

hipError_t launch_exchange(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status, const void* src,
                           void* dst, bool reverse, bool first, int vec, hipStream_t st) {
    const int64_t rows = (int64_t)sh.R * sh.TK;
    const Split sp = copy_split(sh.row_bytes, vec, rows, sh.num_cu);
    const unsigned grid = (unsigned)((first ? table_blocks(sh.R) : 0) + piece_blocks(rows, sp));
    if (grid == 0) return hipSuccess;
    const int64_t bytes = rows * sh.row_bytes;
    return with_vec(vec, [&](auto B) {
        using V = typename Vec<decltype(B)::value>::T;
        return with_unroll(sp.cv, [&](auto U) {
            return with_nt(bytes, [&](auto NT) {
                constexpr int u = decltype(U)::value;
                constexpr bool nt = decltype(NT)::value;
                constexpr unsigned lds = nt ? kCopyLds : 0u;   // streaming: two blocks per CU
                if (first)
                    hipLaunchKernelGGL((exchange_kernel<V, u, nt, false, true, kRowsPerBlock>), dim3(grid),
                                       dim3(kBlock), lds, st, (const V*)src, (V*)dst, sh, tb, out, status, sp);
                else if (reverse)
                    hipLaunchKernelGGL((exchange_kernel<V, u, nt, true, false, kRowsPerBlock>), dim3(grid),
                                       dim3(kBlock), lds, st, (const V*)src, (V*)dst, sh, tb, out, status, sp);
                else if (!sh.layout && nt)   // streaming sizes only: at decode sizes the extra
                                             // dependent search made the staged step 8 % slower
                    hipLaunchKernelGGL((exchange_recv_order_kernel<V, u, nt, kRowsPerBlock>), dim3(grid), dim3(kBlock),
                                       lds, st, (const V*)src, (V*)dst, sh, tb, status, sp);
                else
                    hipLaunchKernelGGL((exchange_kernel<V, u, nt, false, false, kRowsPerBlock>), dim3(grid),
                                       dim3(kBlock), lds, st, (const V*)src, (V*)dst, sh, tb, out, status, sp);
                return hipGetLastError();
            });
        });
    });
}

template <int B, int DT>
static hipError_t launch_combine_t(const Shape& sh, const Tables& tb, const void* rows, const float* gates, void* y,
                                   uint32_t* status, bool direct, hipStream_t st) {
    using V = typename Vec<B>::T;
    const int64_t N = (int64_t)sh.R * sh.T;
    const int64_t bytes = N * sh.row_bytes;
    // at streaming sizes every row is cut in (at least) two pieces, one wavefront each:
    // same-box A/B, prefill combine 227.5 -> 222.2 us staged and 229.9 -> 221.3 us direct,
    // top-8 782 -> 738 us staged and 811 -> 766 us direct (four pieces: 775 / 799 us).
    // The copy kernels cut only long rows (copy_split): shorter ones were slower cut.
    const Split sp = make_split(sh.row_bytes, B, N, sh.num_cu, kCombineWavesPerCu, bytes >= kStreamBytes ? 2 : 1);
    return with_unroll(sp.cv, [&](auto U) {
        return with_nt(bytes, [&](auto NT) {
            // keep float accumulators and the two slots' rows within a sane register
            // budget: 64 accumulators for one slot, 32 when slots are double-buffered
            constexpr int NE = Elems<B, DT>::N, U0 = decltype(U)::value;
            constexpr int U1 = U0 * NE > 64 ? 64 / NE : U0, UK = U0 * NE > 32 ? 32 / NE : U0;
            constexpr bool nt = decltype(NT)::value;
            constexpr int rpb = kRowsPerBlock;   // measured: 1024-thread blocks make the combine ~6 % slower
            const unsigned grid = (unsigned)((N * sp.cpr + rpb - 1) / rpb);
            const dim3 block(rpb * kWave);
            if (sh.k == 1) {
                if (direct)
                    hipLaunchKernelGGL((combine_kernel<B, DT, U1, nt, true, false, rpb>), dim3(grid), block, 0, st,
                                       (const V*)rows, gates, (V*)y, sh, tb, status, sp);
                else
                    hipLaunchKernelGGL((combine_kernel<B, DT, U1, nt, false, false, rpb>), dim3(grid), block, 0, st,
                                       (const V*)rows, gates, (V*)y, sh, tb, status, sp);
            } else {
                if (direct)
                    hipLaunchKernelGGL((combine_kernel<B, DT, UK, nt, true, true, rpb>), dim3(grid), block, 0, st,
                                       (const V*)rows, gates, (V*)y, sh, tb, status, sp);
                else
                    hipLaunchKernelGGL((combine_kernel<B, DT, UK, nt, false, true, rpb>), dim3(grid), block, 0, st,
                                       (const V*)rows, gates, (V*)y, sh, tb, status, sp);
            }
            return hipGetLastError();
        });
    });
}

hipError_t launch_combine(const Shape& sh, const Tables& tb, const void* rows, const float* gates, void* y,
                          uint32_t* status, bool direct, int vec, hipStream_t st) {
    if ((int64_t)sh.R * sh.T == 0) return hipSuccess;
    if (sh.dtype == 1) {
        switch (vec) {
            case 16: return launch_combine_t<16, 1>(sh, tb, rows, gates, y, status, direct, st);
            case 8: return launch_combine_t<8, 1>(sh, tb, rows, gates, y, status, direct, st);
            case 4: return launch_combine_t<4, 1>(sh, tb, rows, gates, y, status, direct, st);
            default: return launch_combine_t<2, 1>(sh, tb, rows, gates, y, status, direct, st);
        }
    }
    switch (vec) {
        case 16: return launch_combine_t<16, 0>(sh, tb, rows, gates, y, status, direct, st);
        case 8: return launch_combine_t<8, 0>(sh, tb, rows, gates, y, status, direct, st);
        default: return launch_combine_t<4, 0>(sh, tb, rows, gates, y, status, direct, st);
    }
}

template <int B, int DT>
static hipError_t launch_expert_t(const Shape& sh, const Tables& tb, const void* in, void* out, int mode,
                                  hipStream_t st) {
    using V = typename Vec<B>::T;
    const int64_t rows = (int64_t)sh.R * sh.TK;
    const Split sp = make_split(sh.row_bytes, B, rows, sh.num_cu);
    return with_unroll(sp.cv, [&](auto U) {
        hipLaunchKernelGGL((expert_kernel<B, DT, decltype(U)::value>), dim3(piece_blocks(rows, sp)), dim3(kBlock), 0,
                           st, (const V*)in, (V*)out, sh, tb, sp, mode);
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

hipError_t launch_reference_copy(const void* src, void* dst, int64_t rows, int64_t row_bytes, int num_cu,
                                 hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const Split sp = copy_split(row_bytes, 16, rows, num_cu);
    return with_unroll(sp.cv, [&](auto U) {
        return with_nt(rows * row_bytes, [&](auto NT) {
            constexpr bool nt = decltype(NT)::value;
            constexpr int rpb = kRowsPerBlock;
            hipLaunchKernelGGL((reference_copy_kernel<decltype(U)::value, nt, rpb>),
                               dim3((unsigned)((rows * sp.cpr + rpb - 1) / rpb)), dim3(rpb * kWave), 0, st,
                               (const u32x4*)src, (u32x4*)dst, rows, sp);
            return hipGetLastError();
        });
    });
}

hipError_t launch_route_step(const int32_t* ids_table, const float* gates_table, int32_t steps, int64_t n,
                             int32_t* counter, int32_t* ids, float* gates, hipStream_t st) {
    hipLaunchKernelGGL(route_step_kernel, dim3(1), dim3(1024), 0, st, ids_table, gates_table, steps, n, counter, ids,
                       gates);
    return hipGetLastError();
}

}  // namespace a2av
