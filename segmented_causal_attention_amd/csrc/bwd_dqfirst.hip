// The backward kernel with the dQ role's workgroups dispatched first (see
// the end of bwd.hip), in a translation unit of its own.
#define SEGATTN_BWD_DQ_FIRST
#include "bwd.hip"
