// Relay split of an uneven grid of serial jobs (shared by the forward and
// backward kernels whose workgroups each run one recurrence through time).
//
// A grid of n equal jobs on m compute units, whose workgroups all stay
// resident, finishes after ceil(n/m) job lengths even when n/m is 1.25 or
// 2.5.  The relay keeps floor(n/m) whole jobs per unit and cuts each of the
// remaining n mod m jobs in time into k = m / (n mod m) pieces, one per unit
// that has room.  Piece j + 1 starts from the state piece j ends with
// (forward in time, or backward for the adjoint): piece j stores it with
// agent-scope atomic stores, waits for them to complete and raises a per-job
// flag; piece j + 1 waits for the flag (acquire) and then reads the state;
// the last piece puts the flag back to zero.  Block
// numbers put every whole job first and then the
// pieces in chain order, and the dispatcher hands out workgroups in number
// order, so a piece that waits was dispatched after the piece it waits for,
// and that one never waits on anything later: every wait ends.  Pieces raise
// their wave priority so that each chain, which is serial, ends with the
// whole jobs that share its units.  A wait is still bounded; if the bound
// runs out, SSM_DEVERR_RELAY is set in the error word.  The split changes no
// arithmetic: pieces start on tile boundaries and pass on every running
// value, so results are bitwise those of the unsplit grid.  Setting the
// environment variable SSM_RELAY to 0 turns the split off (for callers that
// share the device with other work, where the units may not hold the grid).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

struct RelaySplit {
    int full = 0;  // blocks [0, full) are whole jobs
    int rem = 0;   // jobs cut into pieces (job full + j for j < rem)
    int k = 0;     // pieces per cut job; 0: no relay
    int len = 0;   // tokens per piece (a multiple of tile)
};

// Host: the split for `jobs` jobs of L tokens, pieces a multiple of `tile`
// tokens, `cap` resident workgroups per compute unit, n_cu units, at most
// max_jobs cut jobs (the workspace's room).  k == 0 when the jobs divide
// evenly, the units cannot hold one more workgroup, or pieces would be
// shorter than a tile.
RelaySplit relay_split(int64_t jobs, int64_t L, int tile, int cap, int n_cu, int max_jobs);

// Round split, for workgroups too large to share a compute unit with the
// relay's extra piece (one resident workgroup per unit): n jobs on s
// resident slots run in ceil(n/s) rounds, so 320 jobs on 256 units take two
// rounds for 1.25 rounds of work.  Every job is cut into k pieces of `len`
// steps, numbered piece-major (block b: piece b / n of job b % n, piece 0
// the first in the job's own order), so that pieces fill the rounds evenly;
// piece j + 1 of a job was dispatched n blocks after piece j and waits on it
// as in the relay above (every wait ends).  k is chosen by a model of the
// time, max(ceil(n k / s), k) rounds of (len + 1) steps (one step for the
// hand-over), over k = 1 .. 8 with len >= min_len; k == 1: no split.
struct RoundSplit {
    int k = 0;    // pieces per job; 0 or 1: no split
    int len = 0;  // steps per piece
};
RoundSplit round_split(int64_t jobs, int steps, int64_t slots, int min_len);

// Host: compute units of the current device, 0 without one (cached).
int device_cus();

// Host: resident workgroups per compute unit for kernel fn at `threads`
// threads and no dynamic LDS on the current device, 0 on error (cached).
int resident_blocks(const void* fn, int threads);

// Block b of a relay grid: the job it runs and its piece (-1: whole job).
struct RelayBlock {
    int job, piece, cut;  // cut: index of the cut job (piece >= 0)
};
__device__ __forceinline__ RelayBlock relay_block(int b, int full, int rem) {
    if (b < full) return RelayBlock{b, -1, 0};
    const int pb = b - full, piece = pb / rem, cut = pb - piece * rem;
    return RelayBlock{full + cut, piece, cut};
}

// Wait until *flag >= want: thread 0 polls, the barrier holds the other
// threads, and each wave's agent-scope acquire fence then makes the stores
// the flag publishes visible to its loads.  Every thread of the workgroup
// must call it.
__device__ __forceinline__ void relay_wait(const int* flag, int want, uint32_t* err) {
    if (threadIdx.x == 0) {
        constexpr int kSpinMax = 1 << 24;  // about ten seconds of polls
        int n = 0;
        while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < want) {
            if (++n == kSpinMax) {
                atomicOr(err, (uint32_t)SSM_DEVERR_RELAY);
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Hand-over values stored for another compute unit: agent-scope atomic
// stores, which go past this unit's L2 without a writeback of the whole
// cache, so that relay_publish_puts needs no release fence.
__device__ __forceinline__ void relay_put(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish values stored with relay_put only: each thread waits until its own
// stores are complete (vmcnt(0); expcnt and lgkmcnt left at their maxima),
// the barrier gathers the workgroup, and thread 0 raises the flag with
// another agent-scope store.  Every thread of the workgroup must call it,
// after its own relay_put stores.  An agent-scope release fence would do the
// same and also write back every dirty line of the unit's L2, which a
// write-heavy kernel pays for at every hand-over (the Mamba-2 backward's
// split measured 1.77 ms with it, 1.43 ms without).
__device__ __forceinline__ void relay_publish_puts(int* flag, int value) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last piece of a chain, once its wait has ended: put the flag back to
// zero, so that a finished call leaves every flag of its workspace at zero
// and the next call can start from there (workspaces start zeroed).
__device__ __forceinline__ void relay_reset(int* flag) {
    if (threadIdx.x == 0) __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ssm
