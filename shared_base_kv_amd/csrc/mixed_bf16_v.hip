// Decode + prefill grid variants with a value adapter only: the mixed source
// compiled once more for them (see the head of mixed_bf16.hip).
#define LRA_MIXED_PART 1
#include "mixed_bf16.hip"
