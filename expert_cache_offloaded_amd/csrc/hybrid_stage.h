// Layout of a hybrid stage: the pinned host memory that one decode layer call shares
// between the GPU (split and merge kernels) and the host branch (the worker pool's
// dispatcher thread).  Plain C++: included by the HIP side and the host side.
//
//   StageHeader  written on the host when the stage is first used (static per stage)
//   StageReq     written by the split kernel for every call: inputs are in place
//   StageDone    written by the host branch: its partial is in y
//   x bf16 [T][H] | host_ids int32 [T][k] | w fp32 [T][k] | y fp32 [T][H]
//
// The request and completion words sit on lines of their own, so each line has one
// writer.  Sequence numbers count calls: a call is submitted when req.seq moves past
// done.seq and complete when done.seq catches up.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mc.h"

namespace mc {

constexpr uint32_t kStageMagic = 0x6d634859u;   // "mcHY"

struct StageHeader {
  uint32_t magic;
  int32_t T, k, E, H;
  mc_banks host;
  mc_host_pool* pool;
  uint64_t off_req, off_done, off_x, off_ids, off_w, off_y;
};

struct StageReq {
  uint64_t seq;       // calls submitted on this stage
  int32_t layer;      // this call's layer
  int32_t ntok;       // this call's valid token count
  uint32_t err;       // merge waits that ran out (sticky)
};

struct StageDone {
  uint64_t seq;       // calls whose host partial is complete
};

inline size_t stage_align(size_t v) { return (v + 255) & ~(size_t)255; }

inline void stage_layout(int T, int k, int H, StageHeader* h, size_t* total) {
  size_t o = stage_align(sizeof(StageHeader));
  h->off_req = o;
  o = stage_align(o + sizeof(StageReq));
  h->off_done = o;
  o = stage_align(o + sizeof(StageDone));
  h->off_x = o;
  o = stage_align(o + (size_t)T * H * 2);
  h->off_ids = o;
  o = stage_align(o + (size_t)T * k * 4);
  h->off_w = o;
  o = stage_align(o + (size_t)T * k * 4);
  h->off_y = o;
  o = stage_align(o + (size_t)T * H * 4);
  *total = o;
}

// host side (host.cpp): the dispatcher of `pool` serves this stage from now on
void host_pool_add_stage(mc_host_pool* pool, StageHeader* stage);
// removes the stage from every dispatcher (waits until none is using it)
void host_pool_drop_stage(StageHeader* stage);

}  // namespace mc
