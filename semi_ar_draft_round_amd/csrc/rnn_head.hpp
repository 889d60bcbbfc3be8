// The RNN head's arguments as the sampler passes them between its steps.
#pragma once
#include <stdint.h>

namespace dspark {

// Splits of the projection's inner dimension (2r + d) across work groups.
constexpr int kRnnSplits = 8;

struct RnnHead {
  const void* W;   // [3r][2r + d] storage type: gate, candidate and output rows
  const void* h;   // [R][gamma][d] storage type: the backbone's hidden states
  int d;
  float* s;        // [R][gamma][r] f32 out: the state after each position
  void* o;         // [R][gamma][r] storage type out: each position's bias vector
  float* part;     // [kRnnSplits][R][3r] f32 workspace: projection partials
};

}  // namespace dspark
