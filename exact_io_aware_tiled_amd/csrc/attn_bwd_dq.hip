// The dQ kernel of the backward pass (alphabetamath.cc, Algorithm "Exact tiled
// softmax attention with block-recomputed vector-Jacobian products", reverse
// procedure), compiled apart from the rest of attn_bwd.hip so that it can take
// its own machine-scheduler strategy.
#define EIAT_BWD_DQ_UNIT 1
#include "attn_bwd.hip"
