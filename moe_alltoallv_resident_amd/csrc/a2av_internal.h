// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace a2av {

// Problem shape, fixed at handle creation.
struct Shape {
    int32_t R;          // virtual ranks
    int32_t T;          // tokens per rank
    int32_t k;          // top-k
    int32_t E;          // experts
    int32_t epr;        // experts per rank
    int32_t H;          // elements per row
    int32_t dtype;      // 0 f32, 1 bf16
    int32_t nbits;      // bits needed to tell experts apart: ceil(log2(E))
    int64_t TK;         // T * k, send rows per rank
    int64_t cap;        // receive rows per rank
    int64_t row_bytes;  // H * element bytes
    int32_t num_cu;     // compute units of the device (sizes row splitting)
    int32_t layout;     // 0 source-major receive buffers, 1 expert-major
};

// Device tables in the handle's workspace (rank-major, int32 rows).
struct Tables {
    int32_t* pos;          // [R][TK]   place of each (token, slot) in its rank's send order, -1 dropped
    int32_t* cnt;          // [R][E]    rows per (source rank, expert)
    int32_t* send_off;     // [R][R+1]  segment starts in each send buffer
    int32_t* recv_counts;  // [R][R]    [dst][src]
    int32_t* recv_off;     // [R][R+1]  [dst][src] exclusive prefix over src, [dst][R] total
    int32_t* eoff;         // [R][E+1]  first place of each expert in the sender's order
    int32_t* xbase;        // [R][E]    expert-major: receive place of (sender, expert)'s first row
    int32_t* recv_eoff;    // [R][epr+1] expert-major: where each local expert's rows start
    int64_t* dest;         // [R][TK]   direct path: receive row d * cap + q of each (token, slot), -1 none
    int32_t* inv;          // [R][TK]   top-1 only: the token at each send place (places past the
                           //           rows sent are not written)
};

// Optional copies of the tables for the caller (any may be null).
struct Outputs {
    int32_t* split;
    int32_t* recv_counts;
    int32_t* recv_off;
};

// Byte width of the vector used for row copies: the largest of 16, 8, 4, 2 dividing
// the row size and the alignment of every base address involved.
int pick_vec_bytes(int64_t row_bytes, const void* const* ptrs, int nptrs);

// Wavefronts per planning block for E experts when LDS holds (waves + rows) * E counters.
int plan_waves(int32_t E, int rows);

hipError_t launch_plan(const Shape& sh, const Tables& tb, const int32_t* ids, const Outputs& out,
                       uint32_t* status, hipStream_t st);
hipError_t launch_plan_from_counts(const Shape& sh, const Tables& tb, const int32_t* send_counts,
                                   uint32_t* status, hipStream_t st);
// Small steps (decode sizes): planning, receiver tables (and expert-major places) and
// the pack in one launch in which every block works from the ids alone.
bool small_dispatch(const Shape& sh, bool direct);
hipError_t launch_dispatch_small(const Shape& sh, const Tables& tb, const int32_t* ids, const Outputs& out,
                                 uint32_t* status, const void* x, void* dst, bool direct, int vec, hipStream_t st);
// Whether pack runs in gather form (one wavefront per send place, reading the token the
// planner put there; top-1 only, where it moves no more bytes than the scatter form, and
// only at streaming sizes).  Planning writes `inv` exactly when this holds.
bool gather_pack(const Shape& sh);
// pack: staged (dst = send buffer) or direct (dst = receive buffer); also builds the
// receive tables (and the caller's copies in `out`) and, for expert-major buffers, the
// expert-major places.
hipError_t launch_pack(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status, const void* x,
                       void* dst, bool direct, int vec, hipStream_t st);
// exchange: forward (send -> recv) or reverse (recv layout -> send places); `first`
// when it directly follows planning (builds the receive tables itself).
hipError_t launch_exchange(const Shape& sh, const Tables& tb, const Outputs& out, uint32_t* status,
                           const void* src, void* dst, bool reverse, bool first, int vec, hipStream_t st);
// combine: rows = return buffer (staged) or expert outputs in the receive layout (direct).
hipError_t launch_combine(const Shape& sh, const Tables& tb, const void* rows, const float* gates, void* y,
                          uint32_t* status, bool direct, int vec, hipStream_t st);
hipError_t launch_expert(const Shape& sh, const Tables& tb, const void* in, void* out, int mode, int vec,
                         hipStream_t st);
hipError_t launch_reference_copy(const void* src, void* dst, int64_t rows, int64_t row_bytes, int num_cu,
                                 hipStream_t st);
hipError_t launch_route_step(const int32_t* ids_table, const float* gates_table, int32_t steps, int64_t n,
                             int32_t* counter, int32_t* ids, float* gates, hipStream_t st);

// Dynamic LDS the planning kernel may use, and so the largest expert count: three rows
// of E counters (one wavefront's, the totals and the counts before a chunk) must fit.
constexpr int32_t kPlanLdsBytes = 63 * 1024;
constexpr int32_t kMaxExperts = 4096;
static_assert(3 * 4 * kMaxExperts <= kPlanLdsBytes, "planning LDS budget");
constexpr int32_t kMaxRanks = 1024;
constexpr int32_t kMaxTopK = 64;

// Status bit of the debug build's device-side bounds checks (A2AV_ST_BOUNDS).
constexpr uint32_t kStBounds = 4u;

}  // namespace a2av
