// Decode + prefill grid variants with a key adapter only and without
// adapters: the mixed source compiled once more for them (see the head of
// mixed_bf16.hip).
#define LRA_MIXED_PART 2
#include "mixed_bf16.hip"
