// Large-M kernel instances, bfloat16.
#define W4A16_BF 1
#include "w4a16_large.inc"
