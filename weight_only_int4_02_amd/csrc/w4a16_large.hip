// Large-M kernel instances, fp16.
#define W4A16_BF 0
#include "w4a16_large.inc"
