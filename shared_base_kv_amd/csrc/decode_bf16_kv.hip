// Decode variants with both a key and a value adapter: the decode source
// compiled a second time for them (see the end of decode_bf16.hip).
#define LRA_DECODE_KV_PART
#include "decode_bf16.hip"
