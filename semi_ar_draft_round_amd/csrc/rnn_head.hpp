// The RNN head's arguments as the sampler passes them between its steps.
#pragma once
#include <stdint.h>

namespace dspark {

struct RnnHead {
  const void* W;   // [3r][2r + d] storage type: gate, candidate and output rows
  const void* h;   // [R][gamma][d] storage type: the backbone's hidden states
  int d;
  float* s;        // [R][gamma][r] f32 out: the state after each position
  void* o;         // [R][gamma][r] storage type out: each position's bias vector
  float* part;     // f32 workspace: bf16, the hidden-state partials [splits][R gamma][3r],
                   // summed into the first; fp32, one position's projection [R][3r]
  const float* P;  // [V][3r] f32 or null: W's W1-row columns applied to every W1 row
};

}  // namespace dspark
