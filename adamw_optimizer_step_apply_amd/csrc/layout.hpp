// layout.hpp -- device-side launch metadata shared by the host planner and the
// gfx950 kernels of the fused AdamW step.
//
// A launch processes a list of segments (a tensor, or the part of a tensor that
// falls inside a ZeRO shard).  Each segment is split into chunks; one
// workgroup processes one chunk.  Chunks of the "vector" kind hold a multiple
// of 8 elements whose addresses in every stream are 16-byte aligned, so every
// lane moves whole dwordx4 words; the other kind ("element") covers peeled
// heads and tails and segments whose streams cannot be aligned together.
#pragma once

#include <stdint.h>

#include "adamw.h"

namespace adamw {

constexpr int kStreams = 5;            // param, grad, exp_avg, exp_avg_sq, aux
// Threads per workgroup, per kernel family, with the occupancy caps in
// kernels.hip: the mixed kernels run 256-lane workgroups, two per CU (8 waves);
// the VALU-heavier pure-bf16 family 256-lane workgroups, four per CU (16 waves);
// the overflow check 256-lane workgroups at full occupancy (it only reads).
// Chosen by interleaved A/B runs on MI355X (OPT-1.3B list, state in the blocked
// layout and per tensor): for the pure family 256 x 4 and 512 x 2 beat 1024 x 1
// by 5% on blocked state and tie with it per tensor; for the mixed family
// 256 x 2 leads every other shape tried, by 0-10% on blocked state.  The chunk
// and tile shapes below assume these sizes.
#ifndef ADAMW_BLOCK_MIXED
#define ADAMW_BLOCK_MIXED 256
#endif
#ifndef ADAMW_BLOCK_PURE
#define ADAMW_BLOCK_PURE 256
#endif
constexpr int kBlockMixed = ADAMW_BLOCK_MIXED;
constexpr int kBlockPure = ADAMW_BLOCK_PURE;
constexpr int kBlockCheck = 256;
constexpr int kPack = 8;               // elements per lane per dwordx4 of a 16-bit stream
constexpr uint32_t kVecBit = 0x80000000u;
constexpr uint32_t kCountMask = 0x7fffffffu;
constexpr int64_t kElemChunkElems = 4096;       // element chunk
// An update kernel's chunk is shared by kXcdParts workgroups, consecutive in
// launch order, so one on each XCD (the dispatcher hands workgroup b to XCD
// b % 8).  The chunk is cut into tiles of packs; tile t goes to part t % 8, and
// each lane of a part takes one 8-element pack per 2048 packs of the chunk.
// All XCDs thus sweep one contiguous region together.  On MI355X (OPT-1.3B
// list, against giving each XCD one contiguous run of 2048-element chunks)
// this streamed the mixed step 7 % faster on blocked state (16384-element
// blocks) and 4-6.5 % per tensor, and the Kahan step 1 % faster blocked and
// 5-9 % per tensor; only the split-master step on blocked state lost (4 %),
// before its master split became branch-free.  Tile sizes, from interleaved
// A/B runs: 256 elements (1 KiB of an fp32 stream) for the mixed step, whose
// param stream is written only, and for the split-master step (ahead of 512
// by 0.7 points of peak on blocked state, 2.2 per tensor); 512 elements
// (1 KiB of a 16-bit param) for the pure-bf16 family, 1-2 % ahead of 256
// there.  Smaller and larger tiles (64-128, 512-1024 elements for the mixed
// step; 256 and 1024-2048 for Kahan) were slower.
constexpr int kXcdParts = 8;
#ifndef ADAMW_TILE_PACKS_MIXED
#define ADAMW_TILE_PACKS_MIXED 32
#endif
#ifndef ADAMW_TILE_PACKS_SPLIT
#define ADAMW_TILE_PACKS_SPLIT 32
#endif
#ifndef ADAMW_TILE_PACKS_PURE
#define ADAMW_TILE_PACKS_PURE 64
#endif
#ifndef ADAMW_TILE_PACKS_PURE_WIDE
#define ADAMW_TILE_PACKS_PURE_WIDE ADAMW_TILE_PACKS_PURE
#endif
constexpr int kTilePacksMixed = ADAMW_TILE_PACKS_MIXED;
constexpr int kTilePacksSplit = ADAMW_TILE_PACKS_SPLIT;
constexpr int kTilePacks = ADAMW_TILE_PACKS_PURE;
constexpr int kTilePacksPureWide = ADAMW_TILE_PACKS_PURE_WIDE;   // fp32 exp_avg and exp_avg_sq + compensation
// The pack of a chunk taken by lane tid of part `part` (per kXcdParts * block
// packs): tile t of p packs belongs to part t % kXcdParts, so
//     ((tid / p) * kXcdParts + part) * p + tid % p,
// a bijection of (part, tid) onto [0, kXcdParts * block) whenever p divides
// the workgroup size.
constexpr uint32_t tile_pack(uint32_t tid, uint32_t part, uint32_t p)
{
    return ((tid / p) * kXcdParts + part) * p + tid % p;
}
// Default vector chunk of an update kernel: one pack per lane of each part.
constexpr int64_t update_chunk_elems(int block) { return (int64_t)kXcdParts * block * kPack; }
// Blocked state: elements per block, one update chunk (every mode).
constexpr int64_t kStateBlockElems = ADAMW_STATE_BLOCK_ELEMS;
static_assert(kStateBlockElems % update_chunk_elems(kBlockMixed) == 0 &&
                  kStateBlockElems % update_chunk_elems(kBlockPure) == 0,
              "a state block holds whole default chunks");
// The overflow check moves 2 B per element (the step 18-28 B): one workgroup
// per chunk, each lane reading this many packs in one pass, so that a
// workgroup's fixed cost (two dependent table loads) is spread over as many
// bytes as a step workgroup moves.
#ifndef ADAMW_CHECK_CHUNK_MULT
#define ADAMW_CHECK_CHUNK_MULT 8
#endif
constexpr int kCheckChunkMult = ADAMW_CHECK_CHUNK_MULT;
constexpr int64_t kCheckChunkElems = (int64_t)kBlockCheck * kPack * kCheckChunkMult;
// A launch's grid counts at most 2^32 - 1 lanes: the chunk limit of a plan
// follows from the lanes one chunk takes (kXcdParts workgroups of an update
// kernel, one check workgroup).
constexpr int kMaxUpdateBlock = kBlockMixed > kBlockPure ? kBlockMixed : kBlockPure;
constexpr int64_t kMaxUpdateChunks = (int64_t)UINT32_MAX / ((int64_t)kXcdParts * kMaxUpdateBlock);
constexpr int64_t kMaxCheckChunks = (int64_t)UINT32_MAX / kBlockCheck;
// The state copy (setup and checkpoint) runs one 256-lane workgroup per chunk.
constexpr int kBlockCopy = 256;
constexpr int64_t kMaxCopyChunks = (int64_t)UINT32_MAX / kBlockCopy;

// Workgroup b of a grid of nb -> the chunk it processes.  The dispatcher hands
// workgroup b to XCD b % 8 (the MI355X has 8 XCDs, each with its own L2); this
// map lets XCD x walk one contiguous run of chunks, so the workgroups in flight
// on an XCD stream neighbouring addresses.  XCD x receives the q + (x < r)
// workgroups b = 8j + x < nb (q = nb / 8, r = nb % 8) and owns as many chunks,
// starting at x*q + min(x, r): a bijection on [0, nb) for every nb.  Plain
// constexpr code, so that the kernels and a host-side test share it.
constexpr uint32_t xcd_chunk(uint32_t b, uint32_t nb)
{
    return (b & 7u) * (nb >> 3) + ((b & 7u) < (nb & 7u) ? (b & 7u) : (nb & 7u)) + (b >> 3);
}

// Update kernels, by launch id.  The pure-bf16 family adds
// 4 * (fp32 exp_avg) + 2 * (fp32 exp_avg_sq) + (bf16 Kahan compensation) to
// kKernelPure; with an fp32 compensation buffer, 2 * (fp32 exp_avg) + (fp32
// exp_avg_sq) to kKernelPureC32.
constexpr int kKernelMixedBf16 = 0;
constexpr int kKernelMixedF16 = 1;
constexpr int kKernelSplit = 3;
constexpr int kKernelPure = 4;
constexpr int kKernelKahan = kKernelPure + 1;   // bf16 moments + compensation
constexpr int kKernelPureC32 = kKernelPure + 8;

// One segment: the device address of its element 0 in each stream (0 for a
// stream the launch does not touch).
struct alignas(64) DevSeg {
    uint64_t ptr[kStreams];
    uint64_t pad[3];
};

// One workgroup's work: elements [off, off + count) of segment `seg`;
// kVecBit in n_kind marks the vector kind.
struct alignas(16) DevChunk {
    uint32_t seg;
    uint32_t n_kind;
    uint64_t off;
};

// One piece of a state copy between the blocked buffer and per-tensor (or flat)
// state buffers: the address of the piece's first element on each side, per
// state stream (exp_avg, exp_avg_sq, aux; 0 for a stream the step does not use).
struct alignas(64) DevCopySeg {
    uint64_t tensor_side[3];
    uint64_t blocked_side[3];
    uint64_t pad[2];
};

// Scalars of one step, written by the prologue kernel and read by the update
// kernel on the same stream.
struct alignas(64) LaunchScalars {
    int32_t skip;        // nonzero: the step is not taken, nothing is written
    int32_t t;           // 1-based index of the step taken
    float step_size;     // lr / (1 - beta1^t)
    float rbc2;          // 1 / (1 - beta2^t)
    float decay;         // 1 - lr*wd
    float lrwd;          // lr*wd
    float omb1;          // 1 - beta1 (fp32)
    float omb2;          // 1 - beta2 (fp32)
    float beta1;
    float beta2;
    float eps;
    float inv_scale;
};

constexpr int64_t kScalarsBytes = 256;
// Counts of finished workgroups of a single-launch step, after the scalars in
// the same workspace block: kDoneLanes first-level counters (workgroup b counts
// in lane b % kDoneLanes) and one second-level counter, each in its own
// 256-byte line so that their atomics do not queue on one address.  All are
// zero between launches.
constexpr int kDoneLanes = 32;
constexpr int64_t kDoneStrideWords = 64;
constexpr int64_t kDoneOffset = kScalarsBytes;
constexpr int64_t kDoneWords = (kDoneLanes + 1) * kDoneStrideWords;
constexpr int64_t kWorkspaceBytes = kDoneOffset + kDoneWords * 4;

// Default largest grid, in workgroups, that runs as a single launch.  Measured
// on MI355X (mixed step, one tensor, pipelined steps): the single launch takes
// 28-32 % off a step of 64k-256k elements, 7 % at 1M and 2 % at 4M, and ties
// from 8M (4096 workgroups) up, where the prologue launch no longer shows.
constexpr int64_t kSingleLaunchMaxWorkgroups = 4096;

// A single-launch step: the update kernel forms the step's scalars itself in
// every workgroup, and the last workgroup to finish stores the advanced counter.
struct FusedStep {
    adamw_hparams hp;
    int32_t* step;              // the caller's step counter
    const int32_t* found_inf;   // nullable skip flag
    uint32_t* done;             // the finished-workgroup counters (kDoneLanes + 1 lines)
    adamw_loss_scale_state* amp;   // nullable: the device-resident dynamic loss scale
    adamw_loss_scaler scaler;      // its rule (with amp)
};

}  // namespace adamw
