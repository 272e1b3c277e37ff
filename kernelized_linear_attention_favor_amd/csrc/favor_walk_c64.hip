// Causal chunk walk (favor_walk.h) instantiated for chunks of 64 tokens.
#include "favor_walk.h"

namespace favor {
namespace walk {
hipError_t launch_walk_c64(const Args& a, int nw, int nsl, hipStream_t s) { return launch_group_impl<64>(a, nw, nsl, s); }
}  // namespace walk
}  // namespace favor
